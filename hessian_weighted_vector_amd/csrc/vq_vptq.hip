// Second-order error propagation with column sub-vectors (VPTQ page, "The
// Core Algorithm", Algorithm 1).  Columns are quantized left to right in
// blocks of B; a column's M/V sub-vectors take their nearest codebook row
// (plain Euclidean distance); its error E[:,n] = (W[:,n] - What[:,n]) / U[n,n]
// is pushed into the block's later columns at once and into every later
// column at the block's end through U[s:s+B, s+B:].  U is the matrix the
// algorithm reads where the page writes H^-1.
//
// Arithmetic.  The working matrix and the errors are float64, and every
// update is taken in the order and rounding of the algorithm as written: a
// column's error is applied to each later column of its block, column after
// column, as w - e*u (product rounded, then the difference; no fused
// multiply-add), and the block's end adds e*u over the block's columns in
// column order into a float64 sum that is then subtracted.  Every nearest-row
// decision equals the exact float64 direct-form one (lowest index among equal
// distances), so the whole trajectory is the float64 algorithm's, bit for bit.
//
// Layout.  The matrix is transposed into the workspace (row n of Wt is
// column n of W, contiguous), and the quantized matrix and the errors are
// kept transposed too; they are transposed back at the end.
//
// V = 8 (C 16-byte aligned, M % 4 == 0): one launch per column,
//   k_col_step_h16 decides column n-1 (each best certified against a rounding
//                  bound, the rest searched again exactly in float64 over the
//                  chunks that can hold the nearest row) and finishes it (its
//                  value and error, the error's share of the block's later
//                  columns), then searches column n on the fp16 matrix cores
//                  with split operands (expanded form, the codebook prepared
//                  once per call by k_vp_absmax and k_vp_prep); workgroups
//                  split K, and each sub-vector's best and second-best scores
//                  meet in packed 64-bit atomicMin keys of (score bits,
//                  index), each chunk's best score kept beside them;
//   k_col_last     decides and finishes the block's last column.
// Other V, or a codebook that is not 16-byte aligned, two launches per column:
//   k_col_assign   the direct form in float64 on the vector units, one result
//                  per 256-centroid chunk;
//   k_col_finalize merges the chunks in order, writes indices, What and E, and
//                  applies the in-block update to the rows j of the block (a
//                  2D grid over elements and groups of rows).
// Per block: k_block_gemm, Wt[s+B:, :] -= U[s:s+B, s+B:]^T Et[s:s+B, :] in
// float64 on the vector units, each output's sum taken over k in order.
#include "vq_internal.h"

namespace vq {
namespace {

constexpr int kTr = 32;             // transpose tile
constexpr int kAsgThreads = 256;
constexpr int kAsgChunk = 256;      // centroids per assignment workgroup
constexpr int kFinThreads = 256;
constexpr int kFinRows = 16;        // in-block rows per finalize workgroup

// dst [Cc x R] (float64) = src [R x Cc]^T (float32) through a padded LDS tile.
__global__ __launch_bounds__(256) void k_transpose_in(const float* __restrict__ src, int64_t R, int64_t Cc,
                                                      double* __restrict__ dst)
{
    __shared__ float t[kTr][kTr + 1];
    const int64_t r0 = (int64_t)blockIdx.y * kTr, c0 = (int64_t)blockIdx.x * kTr;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    for (int k = ty; k < kTr; k += 8) {
        const int64_t r = r0 + k, c = c0 + tx;
        if (r < R && c < Cc) t[k][tx] = src[r * Cc + c];
    }
    __syncthreads();
    for (int k = ty; k < kTr; k += 8) {
        const int64_t c = c0 + k, r = r0 + tx;
        if (r < R && c < Cc) dst[c * R + r] = (double)t[tx][k];
    }
}

// dst [Cc x R] (float32) = src [R x Cc]^T, src float32 or float64 (rounded to
// nearest float32).
template <class T>
__global__ __launch_bounds__(256) void k_transpose_out(const T* __restrict__ src, int64_t R, int64_t Cc,
                                                       float* __restrict__ dst)
{
    __shared__ float t[kTr][kTr + 1];
    const int64_t r0 = (int64_t)blockIdx.y * kTr, c0 = (int64_t)blockIdx.x * kTr;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    for (int k = ty; k < kTr; k += 8) {
        const int64_t r = r0 + k, c = c0 + tx;
        if (r < R && c < Cc) t[k][tx] = (float)src[r * Cc + c];
    }
    __syncthreads();
    for (int k = ty; k < kTr; k += 8) {
        const int64_t c = c0 + k, r = r0 + tx;
        if (r < R && c < Cc) dst[c * R + r] = t[tx][k];
    }
}

__global__ void k_fill_u64(unsigned long long* __restrict__ p, int64_t n, unsigned long long v)
{
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q < n) p[q] = v;
}

__global__ void k_fill_i32(int* __restrict__ p, int64_t n, int v)
{
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q < n) p[q] = v;
}

// Nearest codebook row of each sub-vector of x (one working column, nv
// sub-vectors of V float64 values, any V) among the workgroup's chunk of
// centroids: the direct form in float64 with the terms added in t order, the
// lowest index among equal distances.  Result per (chunk, sub-vector).
__global__ __launch_bounds__(kAsgThreads) void k_col_assign(const double* __restrict__ x, int nv, int V,
                                                            const float* __restrict__ C, int K,
                                                            double* __restrict__ part_d, int* __restrict__ part_i)
{
    __shared__ float cs[kAsgChunk * 8];
    const int k0 = blockIdx.y * kAsgChunk;
    const int kn = K - k0 < kAsgChunk ? K - k0 : kAsgChunk;
    for (int q = threadIdx.x; q < kn * V; q += kAsgThreads) cs[q] = C[(size_t)k0 * V + q];
    __syncthreads();
    const int v = blockIdx.x * kAsgThreads + threadIdx.x;
    if (v >= nv) return;
    double xv[8];
    for (int t = 0; t < 8; ++t) xv[t] = t < V ? x[(size_t)v * V + t] : 0.0;
    double best = __builtin_inf();
    int arg = 0;
    for (int k = 0; k < kn; ++k) {
        double dist = 0.0;
        for (int t = 0; t < V; ++t) {
            const double df = xv[t] - (double)cs[k * V + t];
            dist += df * df;
        }
        if (dist < best) { best = dist; arg = k; }
    }
    part_d[(size_t)blockIdx.y * nv + v] = best;
    part_i[(size_t)blockIdx.y * nv + v] = k0 + arg;
}

// order-preserving bits of a float (finite or infinite)
__device__ inline unsigned sortable(float f)
{
    const unsigned u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline float unsortable(unsigned v)
{
    return __uint_as_float((v & 0x80000000u) ? (v & 0x7FFFFFFFu) : ~v);
}

// V = 8 on the fp16 matrix cores with split operands.  Once per call the
// codebook is scaled by 2^sc (max |c| 2^sc < 2^10) and split into fp16
// c_hi + c_lo, and hn = |c|^2 / 2 at the same scale (2^(2 sc)) times
// 2^-kHnShift is written as three fp16 pieces (k_vp_prep).  Per wavefront of
// 32 sub-vectors, x is scaled by 2^sx (the wave's largest |x| 2^sx < 2^10)
// and split the same way.  For a 32 x 32 tile two v_mfma_f32_32x32x16_f16
//   acc = [c_hi | c_lo].[x_hi | x_hi] + [c_hi | hn pieces].[x_lo | b b b 0 ..]
// with b = -2^(kHnShift + sx - sc) give acc = 2^(sc + sx) (<c, x> - hn), up to
// the dropped c_lo x_lo term (below 2^-22 |c| |x| per element) and float32
// accumulation; the nearest centroid is the largest acc.  Lane l supplies
// k-slots (l / 32) * 8 .. + 8 of row (A: centroid) or column (B: sub-vector)
// l % 32; accumulator r of lane l is centroid (r / 4) * 8 + (l / 32) * 4 +
// r % 4 of the tile.  The workgroup stages kVpChunk prepared centroids in LDS
// and its four wavefronts search them for 32 sub-vectors each.  Each lane
// keeps the largest and second-largest acc it sees; per sub-vector the
// chunk's best enters key A and the chunk's second-best (and every best that
// a smaller key displaces from A) enters key B, both by atomicMin on
// (order-preserving bits of -acc, index), one of kKeySlots copies per chunk:
// afterwards the smallest key over A's copies is the best of all chunks and
// the smallest over the rest is the second best.  Scores of different chunks
// are comparable: the wave grouping of sub-vectors, hence sx, is the same in
// every chunk.
//
// Certification.  With u = 2^-24, the computed score of centroid k differs
// from <c_k, x> - |c_k|^2/2 (x the float64 working values) by at most
//   2^-18 (1.25 |c_k| |x| + 0.625 |c_k|^2 / 2) + beta 2^-(sc+sx):
// each of the two 16-product float32 sums errs by at most 32u of the
// magnitudes it adds (the first: the sum of |c_t x_t|; the second: that again
// plus the norm term), the split drops at most 3 * 2^-22 |c_t x_t| per term,
// and x's rounding to float32 adds u; beta = 2^-8 covers subnormal split parts
// in scaled units.  Without the norm term (its power-of-two factor below
// fp16's range) |c_k|^2 / 2 is added.  Any centroid at least as near as the
// best's has |c_k| <= R = |x| + sqrt(D_best), so when best - second exceeds
// twice that bound at |c_k| = R the best is the exact nearest row, and
// float64 rounding of the direct form (relative 2^-49) cannot reorder it.
// col_certify makes this check at the start of the next launch and
// col_resolve searches the sub-vectors that fail again in float64 (the direct
// form, terms in t order, lowest index on ties) over the chunks that can hold
// the nearest row.
constexpr int kVpChunk = 512;        // centroids per workgroup (prepared codebook is padded to whole chunks)
constexpr int kHnShift = 9;          // hn 2^(2 sc) < 2^22, its pieces below 2^13
constexpr int kStepRows = 128;       // sub-vectors per workgroup of the column step (4 waves x 32)

constexpr int kKeySlots = 4;         // key copies per column: chunk y merges into slot y % kKeySlots

// Key buffers of the V = 8 path: three columns in rotation, each with
// kKeySlots copies of an A and a B key per sub-vector.
__device__ inline size_t key_at(int nv, int slot, int kind, int64_t n, int j)
{
    return (((size_t)(n % 3) * kKeySlots + (size_t)slot) * 2 + (size_t)kind) * (size_t)nv + (size_t)j;
}

// v of another lane by a DPP pattern (every row and bank enabled).
template <int kCtrl>
__device__ inline float dpp_f(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, true));
}

// Largest of v over the lane's half-wavefront (lanes 0-31 or 32-63): DPP
// exchanges inside each row of 16 lanes (quad swaps, then the half-row and
// row mirrors) and one swizzle between the two rows of the half.
__device__ inline float half_max(float v)
{
    v = fmaxf(v, dpp_f<0xB1>(v));                        // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_f<0x4E>(v));                        // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_f<0x141>(v));                       // row_half_mirror
    v = fmaxf(v, dpp_f<0x140>(v));                       // row_mirror
    v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F)));
    return v;
}

typedef float vp_f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 vp_h16x8 __attribute__((ext_vector_type(8)));

// max |C| over K x 8 floats (one workgroup; C 16-byte aligned)
__global__ __launch_bounds__(1024) void k_vp_absmax(const float4* __restrict__ C4, int64_t n4,
                                                    float* __restrict__ cmax)
{
    __shared__ float red[1024];
    float m = 0.0f;
    for (int64_t q = threadIdx.x; q < n4; q += 1024) {
        const float4 c = C4[q];
        m = fmaxf(m, fmaxf(fmaxf(fabsf(c.x), fabsf(c.y)), fmaxf(fabsf(c.z), fabsf(c.w))));
    }
    red[threadIdx.x] = m;
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
        __syncthreads();
    }
    if (threadIdx.x == 0) *cmax = red[0];
}

__device__ inline int vp_scale_exp(float maxabs)
{
    int e;
    frexpf(maxabs, &e);               // maxabs < 2^e (e = 0 for 0)
    return 10 - e;
}

// Prepared codebook: hi[k], lo[k], hn[k] (8 halfs each) for k < Kp (a whole
// number of chunks); rows k >= K are zero and never searched.
__global__ __launch_bounds__(256) void k_vp_prep(const float* __restrict__ C, int K, int Kp,
                                                 const float* __restrict__ cmax, vp_h16x8* __restrict__ hi,
                                                 vp_h16x8* __restrict__ lo, vp_h16x8* __restrict__ hn)
{
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= Kp) return;
    vp_h16x8 h, l, p;
    for (int t = 0; t < 8; ++t) { h[t] = (_Float16)0.0f; l[t] = (_Float16)0.0f; p[t] = (_Float16)0.0f; }
    if (k < K) {
        const int sc = vp_scale_exp(*cmax);
        double nrm = 0.0;
        for (int t = 0; t < 8; ++t) {
            const float c = C[(size_t)k * 8 + t];
            nrm += (double)c * (double)c;
            const float cs = ldexpf(c, sc);
            const _Float16 ch = (_Float16)cs;
            h[t] = ch;
            l[t] = (_Float16)(cs - (float)ch);
        }
        const double v = ldexp(0.5 * nrm, 2 * sc - kHnShift);
        const _Float16 p1 = (_Float16)v;
        const double r1 = v - (double)p1;
        const _Float16 p2 = (_Float16)r1;
        p[0] = p1;
        p[1] = p2;
        p[2] = (_Float16)(r1 - (double)p2);
    }
    hi[k] = h;
    lo[k] = l;
    hn[k] = p;
}

// Per-workgroup state of one column's decisions (V = 8 path): the
// uncertified decisions of each wavefront (a slot per lane of the lower half),
// and the exact winners found for them with their codebook rows.
struct ColDecide {
    int wcnt[4];                     // uncertified decisions per wavefront
    int flag[kStepRows];             // slot wave * 32 + i: the local sub-vector
    int sh[kStepRows];               // its score scale exponent sc + sx
    double sa[kStepRows];            // its computed best score
    double bnd[kStepRows];           // its rounding bound
    int dec[kStepRows];              // exact winner, by local sub-vector
    float4 row[kStepRows][2];        // the winner's codebook row, by local sub-vector
    double wd[4];                    // one exact search: each wavefront's nearest row,
    int wk[4];                       // its index
    float4 wr[4][2];                 // and the row
};

// A column's decisions for the workgroup's kStepRows sub-vectors, in two
// parts around a workgroup barrier that the caller places between them
// (lanes l and l + 32 of a wavefront hold the same sub-vector).
//
// col_certify: the lane's winner from the column's keys, certified as
// described above; an uncertified one is listed in sd (lower half-wave).
// x: the lane's sub-vector of column p in float64 (zero beyond nv).
//
// col_resolve (after the barrier): the listed sub-vectors are searched again
// exactly in float64 (direct form, terms in t order, the lowest index among
// equal distances), one wavefront each, over the candidate chunks only:
// every workgroup of the column wrote its chunk's best score per sub-vector
// (cbest), and a chunk whose best lies more than twice the bound below the
// column's best cannot hold a centroid at least as near as the computed
// winner (its exact scores are below the winner's exact score), so no
// minimizer and no tie is left out.  Every workgroup of the same rows makes
// the same decisions from the same data.  Returns the number of listed
// sub-vectors; kw and qv then hold the lane's winner and its row.
struct ColCert {
    bool ok;
    int kw;
    float qv[8];
};

// The best and second-best keys of the lane's sub-vector in column p (the
// smallest over A's copies; the smallest over the rest and B's copies).
__device__ inline void col_keys(int nv, int64_t p, const unsigned long long* __restrict__ keys,
                                unsigned long long& a1, unsigned long long& k2)
{
    const int j = blockIdx.x * kStepRows + (threadIdx.x >> 6) * 32 + (threadIdx.x & 31);
    a1 = ~0ull;
    k2 = ~0ull;
    if (j < nv) {
        unsigned long long ka[kKeySlots], kb[kKeySlots];
#pragma unroll
        for (int q = 0; q < kKeySlots; ++q) {
            ka[q] = keys[key_at(nv, q, 0, p, j)];
            kb[q] = keys[key_at(nv, q, 1, p, j)];
        }
        unsigned long long a2 = ~0ull, bmin = ~0ull;
#pragma unroll
        for (int q = 0; q < kKeySlots; ++q) {
            if (ka[q] < a1) { a2 = a1; a1 = ka[q]; } else if (ka[q] < a2) { a2 = ka[q]; }
            bmin = kb[q] < bmin ? kb[q] : bmin;
        }
        k2 = a2 < bmin ? a2 : bmin;
    }
}

__device__ inline ColCert col_certify(ColDecide& sd, int nv, const float* __restrict__ C, unsigned long long a1,
                                      unsigned long long k2, float cmv, const double (&x)[8])
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int jl = lane & 31, half = lane >> 5;
    const int local = wave * 32 + jl;
    const int j = blockIdx.x * kStepRows + local;
    ColCert r;
    r.ok = true;
    r.kw = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) r.qv[t] = 0.0f;
    // the wave's scale, as the search of column p formed it
    float mx = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) mx = fmaxf(mx, fabsf((float)x[t]));
    mx = half_max(mx);
    const int sc = vp_scale_exp(cmv);
    const int sx = min(vp_scale_exp(mx), sc + 15 - kHnShift);
    const bool no_norm = kHnShift + sx - sc < -24;       // the search ran without the norm term
    double sA = 0.0, bound = 0.0;
    if (j < nv) {
        r.kw = (int)(a1 & 0xFFFFFFFFull);
        const float4* c4 = reinterpret_cast<const float4*>(C) + 2 * (size_t)r.kw;
        const float4 ca = c4[0], cb = c4[1];
        r.qv[0] = ca.x; r.qv[1] = ca.y; r.qv[2] = ca.z; r.qv[3] = ca.w;
        r.qv[4] = cb.x; r.qv[5] = cb.y; r.qv[6] = cb.z; r.qv[7] = cb.w;
        if (k2 != ~0ull) {
            sA = -(double)unsortable((unsigned)(a1 >> 32));
            const double sB = -(double)unsortable((unsigned)(k2 >> 32));
            double nx2 = 0.0, db = 0.0;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                nx2 += x[t] * x[t];
                const double df = x[t] - (double)r.qv[t];
                db += df * df;
            }
            const double nx = sqrt(nx2) * (1.0 + 0x1p-40);
            const double R = nx + sqrt(db) * (1.0 + 0x1p-40);
            bound = 0x1p-18 * (1.25 * R * nx + 0.3125 * R * R) + ldexp(0x1p-8, -(sc + sx)) + 0x1p-45 * (nx2 + db);
            if (no_norm) bound += 0.5 * R * R;
            const double gap = ldexp(sA - sB, -(sc + sx));
            r.ok = gap > 2.0 * bound;                    // false also for NaN
        }
    }
    const unsigned long long fm = __ballot(half == 0 && !r.ok);
    if (half == 0 && !r.ok) {
        const int slot = wave * 32 + __popcll(fm & ((1ull << lane) - 1));
        sd.flag[slot] = local;
        sd.sh[slot] = sc + sx;
        sd.sa[slot] = sA;
        sd.bnd[slot] = bound;
    }
    if (lane == 0) sd.wcnt[wave] = __popcll(fm);
    return r;
}

__device__ inline int col_resolve(ColDecide& sd, int nv, int64_t p, const double* __restrict__ xcol,
                                  const float* __restrict__ C, int K, const float* __restrict__ cbest, int nch,
                                  ColCert& r)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int total = sd.wcnt[0] + sd.wcnt[1] + sd.wcnt[2] + sd.wcnt[3];
    if (total == 0) return 0;
    // one listed sub-vector at a time, its candidate chunks dealt to the four
    // wavefronts in turn (each wavefront finds the same candidates), all rows
    // of a chunk requested at once; the wavefronts' results meet in LDS
    for (int ww = 0; ww < 4; ++ww) {
        const int cnt = sd.wcnt[ww];
        for (int i = 0; i < cnt; ++i) {
            const int slot = ww * 32 + i;
            const int lj = sd.flag[slot];
            const int jj = blockIdx.x * kStepRows + lj;
            const double sa = sd.sa[slot], twob = 2.0 * sd.bnd[slot];
            const int sh = sd.sh[slot];
            double xv[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) xv[t] = xcol[(size_t)jj * 8 + t];
            double bd = __builtin_inf();
            int bk = 0x7FFFFFFF;
            float4 ra = make_float4(0.0f, 0.0f, 0.0f, 0.0f), rb = ra;
            int seen = 0;                                // candidates met so far (the same in every wavefront)
            for (int c0 = 0; c0 < nch; c0 += 64) {
                bool cand = false;
                if (c0 + lane < nch) {
                    const float cbv = cbest[((size_t)(p & 1) * nch + c0 + lane) * nv + jj];
                    cand = !(ldexp(sa - (double)cbv, -sh) > twob);
                }
                unsigned long long m = __ballot(cand);
                while (m) {
                    const int cc = c0 + __ffsll((long long)m) - 1;
                    m &= m - 1;
                    if ((seen++ & 3) != wave) continue;
                    const int k0 = cc * kVpChunk;
                    const int kn = K - k0 < kVpChunk ? K - k0 : kVpChunk;
                    float4 ca[kVpChunk / 64], cb[kVpChunk / 64];
#pragma unroll
                    for (int u = 0; u < kVpChunk / 64; ++u) {
                        const int q = lane + 64 * u;
                        const float4* c4 = reinterpret_cast<const float4*>(C) + 2 * (size_t)(k0 + (q < kn ? q : 0));
                        ca[u] = c4[0];
                        cb[u] = c4[1];
                    }
#pragma unroll
                    for (int u = 0; u < kVpChunk / 64; ++u) {
                        const int q = lane + 64 * u;
                        const float cv[8] = {ca[u].x, ca[u].y, ca[u].z, ca[u].w, cb[u].x, cb[u].y, cb[u].z, cb[u].w};
                        double dist = 0.0;
#pragma unroll
                        for (int t = 0; t < 8; ++t) {
                            const double df = xv[t] - (double)cv[t];
                            dist += df * df;
                        }
                        const int k = k0 + q;
                        if (q < kn && (dist < bd || (dist == bd && k < bk))) {
                            bd = dist;
                            bk = k;
                            ra = ca[u];
                            rb = cb[u];
                        }
                    }
                }
            }
            // the wavefront's smallest (distance, index); its lane (indices
            // are distinct) leaves it, with the row, for the merge
            double md = bd;
            int mk = bk;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const double od = __shfl_xor(md, o);
                const int oi = __shfl_xor(mk, o);
                if (od < md || (od == md && oi < mk)) { md = od; mk = oi; }
            }
            if (mk == 0x7FFFFFFF ? lane == 0 : (bk == mk && bd == md)) {
                sd.wd[wave] = md;
                sd.wk[wave] = mk;
                sd.wr[wave][0] = ra;
                sd.wr[wave][1] = rb;
            }
            __syncthreads();
            if (threadIdx.x == 0) {
                int w = 0;
#pragma unroll
                for (int v = 1; v < 4; ++v)
                    if (sd.wd[v] < sd.wd[w] || (sd.wd[v] == sd.wd[w] && sd.wk[v] < sd.wk[w])) w = v;
                sd.dec[lj] = sd.wk[w];
                sd.row[lj][0] = sd.wr[w][0];
                sd.row[lj][1] = sd.wr[w][1];
            }
            __syncthreads();
        }
    }
    if (!r.ok) {
        const int local = wave * 32 + (lane & 31);
        r.kw = sd.dec[local];
        const float4 ca = sd.row[local][0], cb = sd.row[local][1];
        r.qv[0] = ca.x; r.qv[1] = ca.y; r.qv[2] = ca.z; r.qv[3] = ca.w;
        r.qv[4] = cb.x; r.qv[5] = cb.y; r.qv[6] = cb.z; r.qv[7] = cb.w;
    }
    return total;
}

// Column n (V = 8 path).  Grid: x over row blocks of kStepRows sub-vectors,
// y over kVpChunk-centroid chunks.  For n past the block's first column it
// first decides column n-1 (col_certify, col_resolve), then finishes it:
// value, error, the error's share of column n (every workgroup of these rows
// forms the same values); the first chunk's workgroups write the outputs,
// and column n-1's error goes into the block's later columns.  Then it
// searches column n over its chunk.  Loads are issued early and their
// registers used late: the previous column's keys first, the chunk written to
// LDS only after the keys and the winners' rows are requested, the later
// column's values at the start.
__global__ __launch_bounds__(256) void k_col_step_h16(
    double* __restrict__ Wt, int64_t M, int nv, int64_t n, int64_t s, int64_t s_end, const float* __restrict__ C,
    const float* __restrict__ U, int64_t N, unsigned long long* __restrict__ keys, float* __restrict__ cbest,
    int nch, double* __restrict__ Xc, uint16_t* __restrict__ idx, float* __restrict__ Wht,
    double* __restrict__ Et, const vp_h16x8* __restrict__ Phi, const vp_h16x8* __restrict__ Plo,
    const vp_h16x8* __restrict__ Phn, const float* __restrict__ cmax, int K, int* __restrict__ fl_total)
{
    static_assert(kVpChunk == 2 * 256, "two prepared centroids per thread");
    __shared__ vp_h16x8 L[3][kVpChunk];
    __shared__ ColDecide sd;
    const int k0 = blockIdx.y * kVpChunk;
    const int kn = K - k0 < kVpChunk ? K - k0 : kVpChunk;
    // the previous column's keys first: the certification waits on them
    unsigned long long ka1 = ~0ull, kk2 = ~0ull;
    if (n > s) col_keys(nv, n - 1, keys, ka1, kk2);
    // the chunk's prepared rows, two centroids per thread (staged in LDS
    // later, after the decision's loads are issued)
    const int ka = k0 + threadIdx.x, kb = ka + 256;
    const vp_h16x8 fa0 = Phi[ka], fa1 = Plo[ka], fa2 = Phn[ka];
    const vp_h16x8 fb0 = Phi[kb], fb1 = Plo[kb], fb2 = Phn[kb];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j0 = (blockIdx.x * 4 + wave) * 32;
    const int jl = lane & 31, half = lane >> 5;
    const int j = j0 + jl;
    const bool active = j0 < nv;                         // the wave holds sub-vectors
    const float cmv = *cmax;
    double x64[8], e[8], w[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        x64[t] = 0.0;
        e[t] = 0.0;
        w[t] = 0.0;
    }
    if (j < nv) {
        const double2* w2 = reinterpret_cast<const double2*>(Wt + n * M) + 4 * (size_t)j;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const double2 v2 = w2[q];
            w[2 * q] = v2.x;
            w[2 * q + 1] = v2.y;
        }
    }
    // the first of the block's later columns that this workgroup updates
    // with column n-1's error (its values requested now, written before the
    // search, so the stores complete while the matrix cores run)
    int64_t rl = n + 1 + blockIdx.y;
    const bool upd = n > s && rl < s_end && j < nv;
    double ul = 0.0, wl[4] = {0.0, 0.0, 0.0, 0.0};
    if (upd) {
        ul = (double)U[(n - 1) * N + rl];
        const double* wr = Wt + rl * M + (int64_t)j * 8 + half * 4;
#pragma unroll
        for (int t = 0; t < 4; ++t) wl[t] = wr[t];
    }
    auto stage = [&]() {
        const int q = threadIdx.x;
        L[0][q] = fa0;
        L[1][q] = fa1;
        L[2][q] = fa2;
        L[0][q + 256] = fb0;
        L[1][q + 256] = fb1;
        L[2][q + 256] = fb2;
    };
    if (n > s) {
        const int64_t p = n - 1;
        const double* xcol = Xc + (size_t)(p & 1) * M;
        double xp[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) xp[t] = j < nv ? xcol[(size_t)j * 8 + t] : 0.0;
        const double unn = (double)U[p * N + p], un = (double)U[p * N + n];
        ColCert r = col_certify(sd, nv, C, ka1, kk2, cmv, xp);
        stage();
        __syncthreads();
        const int nfl = col_resolve(sd, nv, p, xcol, C, K, cbest, nch, r);
        if (j < nv) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                e[t] = (xp[t] - (double)r.qv[t]) / unn;
                x64[t] = w[t] - e[t] * un;
            }
            if (blockIdx.y == 0 && half == 0) {
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    Wht[p * M + (int64_t)j * 8 + t] = r.qv[t];
                    Et[p * M + (int64_t)j * 8 + t] = e[t];
                }
                idx[p * nv + j] = (uint16_t)r.kw;
            }
            // column n-1's error into the block's later columns, split over
            // the workgroups of these rows by column (no later read in this
            // launch)
            if (upd) {
                double* wr = Wt + rl * M + (int64_t)j * 8 + half * 4;
#pragma unroll
                for (int t = 0; t < 4; ++t) wr[t] = wl[t] - e[half * 4 + t] * ul;
                for (rl += gridDim.y; rl < s_end; rl += gridDim.y) {
                    const double ur = (double)U[p * N + rl];
                    double* wq = Wt + rl * M + (int64_t)j * 8 + half * 4;
#pragma unroll
                    for (int t = 0; t < 4; ++t) wq[t] = wq[t] - e[half * 4 + t] * ur;
                }
            }
        }
        if (blockIdx.y == 0 && threadIdx.x == 0 && nfl > 0) atomicAdd(fl_total, nfl);
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) x64[t] = w[t];
        stage();
        __syncthreads();
    }
    if (blockIdx.y == 0 && half == 0 && j < nv) {
#pragma unroll
        for (int t = 0; t < 8; ++t) Xc[(size_t)(n & 1) * M + (size_t)j * 8 + t] = x64[t];
#pragma unroll
        for (int q = 0; q < kKeySlots; ++q) {
            keys[key_at(nv, q, 0, n + 1, j)] = ~0ull;
            keys[key_at(nv, q, 1, n + 1, j)] = ~0ull;
        }
    }
    // the wave's scale (both halves hold the same 32 sub-vectors)
    float xv[8];
    float mx = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        xv[t] = (float)x64[t];
        mx = fmaxf(mx, fabsf(xv[t]));
    }
    mx = half_max(mx);
    const int sc = vp_scale_exp(cmv);
    const int sx = min(vp_scale_exp(mx), sc + 15 - kHnShift);
    const int eb = kHnShift + sx - sc;                  // <= 15: b is a finite fp16
    const _Float16 b = eb >= -24 ? (_Float16)(-ldexpf(1.0f, eb)) : (_Float16)0.0f;
    float best = -__builtin_inff(), sec = -__builtin_inff();
    int bi = 0;
    if (active) {
        vp_h16x8 bh, b2;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float xs = ldexpf(xv[t], sx);
            const _Float16 h = (_Float16)xs;
            bh[t] = h;
            b2[t] = half ? (t < 3 ? b : (_Float16)0.0f) : (_Float16)(xs - (float)h);
        }
        const vp_h16x8* A1 = L[half ? 1 : 0];
        const vp_h16x8* A2 = L[half ? 2 : 0];
        const int ntiles = (kn + 31) / 32;
        // per tile its largest score: the lane's best and second-best tile
        // maxima and the best's tile, whose 16 scores the lane keeps (a
        // select per score, no branch)
        float m1 = -__builtin_inff(), m2 = -__builtin_inff();
        int bt = 0;
        float pk[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) pk[r] = -__builtin_inff();
        auto scan = [&](vp_f32x16 acc, int tb) {
            if (tb + 32 > kn) {                          // the chunk's last, partial tile
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (tb + (r >> 2) * 8 + half * 4 + (r & 3) >= kn) acc[r] = -__builtin_inff();
            }
            float m = fmaxf(fmaxf(acc[0], acc[1]), acc[2]);
#pragma unroll
            for (int r = 3; r < 15; r += 2) m = fmaxf(fmaxf(m, acc[r]), acc[r + 1]);
            m = fmaxf(m, acc[15]);
            m2 = __builtin_amdgcn_fmed3f(m1, m2, m);
            const bool imp = m > m1;
            bt = imp ? tb : bt;
#pragma unroll
            for (int r = 0; r < 16; ++r) pk[r] = imp ? acc[r] : pk[r];
            m1 = fmaxf(m1, m);
        };
        const vp_f32x16 zero = {};
        // the operands of the next tile pair are read before the current
        // pair's scores are scanned
        vp_h16x8 p0 = A1[jl], p1 = A1[32 + jl], q0 = A2[jl], q1 = A2[32 + jl];
        int tb = 0;
        for (; tb + 32 < ntiles * 32; tb += 64) {
            vp_f32x16 a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(p0, bh, zero, 0, 0, 0);
            vp_f32x16 a1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(p1, bh, zero, 0, 0, 0);
            a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(q0, b2, a0, 0, 0, 0);
            a1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(q1, b2, a1, 0, 0, 0);
            if (tb + 64 < kVpChunk) {
                p0 = A1[tb + 64 + jl];
                p1 = A1[tb + 96 + jl];
                q0 = A2[tb + 64 + jl];
                q1 = A2[tb + 96 + jl];
            }
            scan(a0, tb);
            scan(a1, tb + 32);
        }
        if (tb < ntiles * 32) {
            vp_f32x16 a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(p0, bh, zero, 0, 0, 0);
            a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(q0, b2, a0, 0, 0, 0);
            scan(a0, tb);
        }
        // the best tile's scores: the lane's best, its index (lowest on
        // ties) and the tile's own second best; the other tiles' maxima give
        // the rest of the second best
        if (m1 > -__builtin_inff()) {
            const float* rf = pk;
            int rr = 0, ties = 0;
            float t2 = -__builtin_inff();                // largest score below the best
#pragma unroll
            for (int r = 15; r >= 0; --r) {
                if (rf[r] == m1) {
                    rr = r;
                    ++ties;
                } else {
                    t2 = fmaxf(t2, rf[r]);
                }
            }
            best = m1;
            sec = fmaxf(m2, ties > 1 ? m1 : t2);
            bi = bt + (rr >> 2) * 8 + half * 4 + (rr & 3);
        }
        // the two halves of the sub-vector's centroid rows: best with the
        // lower index among equal scores, second best of the four values
        const float ob = __shfl_xor(best, 32), os = __shfl_xor(sec, 32);
        const int oi = __shfl_xor(bi, 32);
        const float lo = fminf(best, ob);
        sec = fmaxf(fmaxf(sec, os), lo);
        if (ob > best || (ob == best && oi < bi)) { best = ob; bi = oi; }
    }
    if (active && half == 0 && j < nv) {
        cbest[((size_t)(n & 1) * nch + blockIdx.y) * nv + j] = fmaxf(best, sec);
        const int slot = blockIdx.y % kKeySlots;
        const unsigned long long kb_ = ((unsigned long long)sortable(-best + 0.0f) << 32) | (unsigned)(k0 + bi);
        const unsigned long long ks_ = ((unsigned long long)sortable(-sec + 0.0f) << 32) | 0xFFFFFFFFull;
        const unsigned long long old = atomicMin(&keys[key_at(nv, slot, 0, n, j)], kb_);
        const unsigned long long lost = old > kb_ ? old : kb_;
        atomicMin(&keys[key_at(nv, slot, 1, n, j)], lost < ks_ ? lost : ks_);
    }
}

// The block's last column n (V = 8 path): its decisions (col_certify,
// col_resolve), value and error; nothing of the block is left to update.
// Grid: row blocks of kStepRows sub-vectors.
__global__ __launch_bounds__(256) void k_col_last(int64_t M, int nv, int64_t n, const float* __restrict__ C, int K,
                                                  const float* __restrict__ U, int64_t N,
                                                  const unsigned long long* __restrict__ keys,
                                                  const float* __restrict__ cbest, int nch,
                                                  const float* __restrict__ cmax, const double* __restrict__ Xc,
                                                  uint16_t* __restrict__ idx, float* __restrict__ Wht,
                                                  double* __restrict__ Et, int* __restrict__ fl_total)
{
    __shared__ ColDecide sd;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int j = blockIdx.x * kStepRows + wave * 32 + (lane & 31);
    const double* xcol = Xc + (size_t)(n & 1) * M;
    double x[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) x[t] = j < nv ? xcol[(size_t)j * 8 + t] : 0.0;
    const double unn = (double)U[n * N + n];
    unsigned long long a1, k2;
    col_keys(nv, n, keys, a1, k2);
    ColCert r = col_certify(sd, nv, C, a1, k2, *cmax, x);
    __syncthreads();
    const int nfl = col_resolve(sd, nv, n, xcol, C, K, cbest, nch, r);
    if (j < nv && half == 0) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            Wht[n * M + (int64_t)j * 8 + t] = r.qv[t];
            Et[n * M + (int64_t)j * 8 + t] = (x[t] - (double)r.qv[t]) / unn;
        }
        idx[n * nv + j] = (uint16_t)r.kw;
    }
    if (threadIdx.x == 0 && nfl > 0) atomicAdd(fl_total, nfl);
}

// Column n (other V): the chunks' winners merged in chunk order (strictly
// smaller distance wins, so the lowest index keeps a tie) -> indices, What,
// E; the block's rows j in (n, s_end) receive w - E[:,n] U[n,j].  Grid: x over
// the M elements, y over groups of kFinRows rows.
__global__ __launch_bounds__(kFinThreads) void k_col_finalize(
    double* __restrict__ Wt, int64_t M, int V, int nv, int64_t n, int64_t s_end, const float* __restrict__ C,
    const float* __restrict__ U, int64_t N, const double* __restrict__ part_d, const int* __restrict__ part_i,
    int nch, uint16_t* __restrict__ idx, float* __restrict__ Wht, double* __restrict__ Et)
{
    const int64_t m = (int64_t)blockIdx.x * kFinThreads + threadIdx.x;
    if (m >= M) return;
    const int v = (int)(m / V);
    const int t = (int)(m - (int64_t)v * V);
    double bd = part_d[v];
    int k = part_i[v];
    for (int c = 1; c < nch; ++c) {
        const double d = part_d[(size_t)c * nv + v];
        if (d < bd) { bd = d; k = part_i[(size_t)c * nv + v]; }
    }
    const float wq = C[(size_t)k * V + t];
    const double e = (Wt[n * M + m] - (double)wq) / (double)U[n * N + n];
    const int64_t j0 = n + 1 + (int64_t)blockIdx.y * kFinRows;
    const int64_t j1 = j0 + kFinRows < s_end ? j0 + kFinRows : s_end;
    for (int64_t j = j0; j < j1; ++j) Wt[j * M + m] = Wt[j * M + m] - e * (double)U[n * N + j];
    if (blockIdx.y == 0) {
        Wht[n * M + m] = wq;
        Et[n * M + m] = e;
        if (t == 0) idx[n * nv + v] = (uint16_t)k;
    }
}

// Wt[s_end + r, m] -= sum_{k < kb} Et[s + k, m] * U[s + k, s_end + r] in
// float64: each output's sum starts at 0 and adds the products (each rounded,
// then added) in k order, then is subtracted.  A 128 (r) x 64 (m) tile per
// workgroup, 8 x 4 outputs per thread; k runs in chunks of kGemmK through
// double-buffered LDS panels (U converted to float64 on the way in; the next
// chunk is loaded into registers while the current one is used).
constexpr int kGemmR = 128;          // output rows (later columns of W) per tile
constexpr int kGemmM = 64;           // output elements per tile
constexpr int kGemmK = 16;           // k per LDS chunk

__global__ __launch_bounds__(256) void k_block_gemm(double* __restrict__ Wt, const float* __restrict__ U,
                                                    const double* __restrict__ Et, int64_t N, int64_t M,
                                                    int64_t s, int kb, int64_t s_end)
{
    __shared__ double As[2][kGemmK][kGemmR];
    __shared__ double Bs[2][kGemmK][kGemmM];
    const int64_t R = N - s_end;
    const int64_t r0 = (int64_t)blockIdx.y * kGemmR, m0 = (int64_t)blockIdx.x * kGemmM;
    const int tid = threadIdx.x;
    // loaders: U panel kGemmK x 128 (8 values per thread), E panel kGemmK x 64 (4 per thread)
    const int ak = tid >> 4, ac = (tid & 15) * 8;
    const int bk = tid >> 4, bc = (tid & 15) * 4;
    double ra[8], rb[4];
    auto load = [&](int kc) {
        const int k = kc + ak;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t r = r0 + ac + i;
            ra[i] = (k < kb && r < R) ? (double)U[(s + k) * N + s_end + r] : 0.0;
        }
        const int k2 = kc + bk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t mm = m0 + bc + i;
            rb[i] = (k2 < kb && mm < M) ? Et[(s + k2) * M + mm] : 0.0;
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; ++i) As[buf][ak][ac + i] = ra[i];
#pragma unroll
        for (int i = 0; i < 4; ++i) Bs[buf][bk][bc + i] = rb[i];
    };
    const int tr = (tid >> 4) * 8, tm = (tid & 15) * 4;
    double acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] = 0.0;
    const int nk = (kb + kGemmK - 1) / kGemmK;
    load(0);
    store(0);
    __syncthreads();
    for (int c = 0; c < nk; ++c) {
        const int buf = c & 1;
        if (c + 1 < nk) load((c + 1) * kGemmK);
        const int kk_end = kb - c * kGemmK < kGemmK ? kb - c * kGemmK : kGemmK;
        for (int kk = 0; kk < kk_end; ++kk) {
            double a[8], bb[4];
#pragma unroll
            for (int i = 0; i < 8; ++i) a[i] = As[buf][kk][tr + i];
#pragma unroll
            for (int q = 0; q < 4; ++q) bb[q] = Bs[buf][kk][tm + q];
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[i][q] = acc[i][q] + bb[q] * a[i];
        }
        if (c + 1 < nk) store(buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t row = r0 + tr + i;
        if (row >= R) continue;
        double* p = Wt + (s_end + row) * M + m0 + tm;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (m0 + tm + q < M) p[q] = p[q] - acc[i][q];
    }
}

}  // namespace

size_t ws_vptq(int64_t M, int64_t N, int V)
{
    const int64_t nv = M / V;
    const int64_t nch = (65536 + kAsgChunk - 1) / kAsgChunk;
    const int64_t nvp = 65536 / kVpChunk;
    // the float64 working matrix and errors, the float32 quantized matrix (all
    // transposed), three key buffers (A and B keys, kKeySlots copies), the
    // chunk best scores of two columns, the count of exact searches, two
    // float64 working columns, the prepared codebook (3 x 16 bytes per
    // centroid, at most 65536), max |C|, and the per-chunk winners of the
    // direct-form search (other V)
    return 2 * align_up((size_t)M * (size_t)N * sizeof(double)) + align_up((size_t)M * (size_t)N * sizeof(float)) +
           align_up((size_t)(3 * kKeySlots * 2 * nv) * sizeof(uint64_t)) +
           align_up((size_t)(2 * nvp * nv) * sizeof(float)) + align_up(sizeof(int)) +
           align_up((size_t)(2 * M) * sizeof(double)) +
           3 * align_up((size_t)65536 * sizeof(vp_h16x8)) + align_up(sizeof(float)) +
           align_up((size_t)(nch * nv) * sizeof(double)) + align_up((size_t)(nch * nv) * sizeof(int));
}

vq_status vptq_launch(const float* W, const float* U, int64_t M, int64_t N, int V, const float* C, int K, int B,
                      uint16_t* idx, float* W_hat, float* E, void* ws, size_t ws_bytes, hipStream_t st)
{
    const int64_t nv = M / V;
    const int64_t nrb = (nv + kStepRows - 1) / kStepRows;
    const int64_t nch_all = (65536 + kAsgChunk - 1) / kAsgChunk;
    const int64_t nvp = 65536 / kVpChunk;
    Carver cv(ws, ws_bytes);
    double* Wt = cv.take<double>((size_t)(M * N));
    double* Et = cv.take<double>((size_t)(M * N));
    float* Wht = cv.take<float>((size_t)(M * N));
    unsigned long long* keys = cv.take<unsigned long long>((size_t)(3 * kKeySlots * 2 * nv));
    float* cbest = cv.take<float>((size_t)(2 * nvp * nv));
    int* fl_total = cv.take<int>(1);
    double* Xc = cv.take<double>((size_t)(2 * M));
    const int Kp = (K + kVpChunk - 1) / kVpChunk * kVpChunk;
    vp_h16x8* Phi = cv.take<vp_h16x8>(65536);
    vp_h16x8* Plo = cv.take<vp_h16x8>(65536);
    vp_h16x8* Phn = cv.take<vp_h16x8>(65536);
    float* cmax = cv.take<float>(1);
    double* part_d = cv.take<double>((size_t)(nch_all * nv));
    int* part_i = cv.take<int>((size_t)(nch_all * nv));
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_vptq: workspace too small");
    TimedRegion tr("vptq", K, st);
    const dim3 tw(grid_for(N, kTr), grid_for(M, kTr));
    hipLaunchKernelGGL(k_transpose_in, tw, dim3(256), 0, st, W, M, N, Wt);
    VQ_LAUNCHED("k_transpose_in");
    const bool v8 = V == 8 && aligned16(C) && (M % 4 == 0);
    if (v8) {
        hipLaunchKernelGGL(k_fill_u64, dim3(grid_for(3 * kKeySlots * 2 * nv, 256)), dim3(256), 0, st, keys,
                           3 * kKeySlots * 2 * nv, ~0ull);
        VQ_LAUNCHED("k_fill_u64");
        hipLaunchKernelGGL(k_fill_i32, dim3(1), dim3(256), 0, st, fl_total, (int64_t)1, 0);
        VQ_LAUNCHED("k_fill_i32");
        hipLaunchKernelGGL(k_vp_absmax, dim3(1), dim3(1024), 0, st, reinterpret_cast<const float4*>(C),
                           (int64_t)K * 2, cmax);
        VQ_LAUNCHED("k_vp_absmax");
        hipLaunchKernelGGL(k_vp_prep, dim3(grid_for(Kp, 256)), dim3(256), 0, st, C, K, Kp, cmax, Phi, Plo, Phn);
        VQ_LAUNCHED("k_vp_prep");
    }
    const int nch = (K + kAsgChunk - 1) / kAsgChunk;
    const dim3 ga(grid_for(nv, kAsgThreads), (unsigned)nch);
    const int nchv = Kp / kVpChunk;
    const dim3 gm((unsigned)nrb, (unsigned)nchv);
    for (int64_t s = 0; s < N; s += B) {
        const int64_t s_end = s + B < N ? s + B : N;
        if (v8) {
            // one launch per column (it also decides and finishes the column
            // before it), and one for the block's last column
            for (int64_t n = s; n < s_end; ++n) {
                hipLaunchKernelGGL(k_col_step_h16, gm, dim3(256), 0, st, Wt, M, (int)nv, n, s, s_end, C, U, N, keys,
                                   cbest, nchv, Xc, idx, Wht, Et, Phi, Plo, Phn, cmax, K, fl_total);
                VQ_LAUNCHED("k_col_step_h16");
            }
            hipLaunchKernelGGL(k_col_last, dim3((unsigned)nrb), dim3(256), 0, st, M, (int)nv, s_end - 1, C, K, U, N,
                               keys, cbest, nchv, cmax, Xc, idx, Wht, Et, fl_total);
            VQ_LAUNCHED("k_col_last");
        } else {
            for (int64_t n = s; n < s_end; ++n) {
                hipLaunchKernelGGL(k_col_assign, ga, dim3(kAsgThreads), 0, st, Wt + n * M, (int)nv, V, C, K, part_d,
                                   part_i);
                VQ_LAUNCHED("k_col_assign");
                const int64_t rows = s_end - n - 1;
                const dim3 gf(grid_for(M, kFinThreads),
                              (unsigned)(rows > 0 ? (rows + kFinRows - 1) / kFinRows : 1));
                hipLaunchKernelGGL(k_col_finalize, gf, dim3(kFinThreads), 0, st, Wt, M, V, (int)nv, n, s_end, C, U,
                                   N, part_d, part_i, nch, idx, Wht, Et);
                VQ_LAUNCHED("k_col_finalize");
            }
        }
        if (s_end < N) {
            TimedRegion tg("vptq_block_update", K, st);
            const dim3 gg(grid_for(M, kGemmM), grid_for(N - s_end, kGemmR));
            hipLaunchKernelGGL(k_block_gemm, gg, dim3(256), 0, st, Wt, U, Et, N, M, s, (int)(s_end - s), s_end);
            VQ_LAUNCHED("k_block_gemm");
        }
    }
    const dim3 tb(grid_for(M, kTr), grid_for(N, kTr));
    hipLaunchKernelGGL(k_transpose_out<float>, tb, dim3(256), 0, st, Wht, N, M, W_hat);
    VQ_LAUNCHED("k_transpose_out");
    if (E) {
        hipLaunchKernelGGL(k_transpose_out<double>, tb, dim3(256), 0, st, Et, N, M, E);
        VQ_LAUNCHED("k_transpose_out");
    }
    if (v8 && timing_on()) {
        // diagnostics: how many decisions the exact search took
        int n_exact = 0;
        VQ_HIP(hipMemcpyAsync(&n_exact, fl_total, sizeof(int), hipMemcpyDeviceToHost, st));
        VQ_HIP(hipStreamSynchronize(st));
        timing_count("vptq_exact_searches", K, n_exact);
    }
    return VQ_OK;
}

}  // namespace vq
