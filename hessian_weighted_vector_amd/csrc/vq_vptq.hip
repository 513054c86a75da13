// Second-order error propagation with column sub-vectors (VPTQ page, "The
// Core Algorithm", Algorithm 1).  Columns are quantized left to right in
// blocks of B; a column's M/V sub-vectors take their nearest codebook row
// (plain Euclidean distance); its error E[:,n] = (W[:,n] - What[:,n]) / U[n,n]
// is pushed into the block's later columns at once and into every later
// column at the block's end through U[s:s+B, s+B:].  U is the matrix the
// algorithm reads where the page writes H^-1.
//
// Layout.  The matrix is transposed into the workspace (row n of Wt is
// column n of W, contiguous), and the quantized matrix and the errors are
// kept transposed too; they are transposed back at the end.
//
// V = 8 (C 16-byte aligned, M % 4 == 0): one launch per column,
//   k_col_step_h16 finishes column n-1 (its winner, value and error, the
//                  error's share of the block's later columns) and searches
//                  column n on the fp16 matrix cores with split operands
//                  (expanded form, the codebook prepared once per call by
//                  k_vp_absmax and k_vp_prep); workgroups split K, and the
//                  per-sub-vector minima meet in a packed 64-bit atomicMin of
//                  (score bits, index): the order of arrival does not matter,
//                  and equal scores keep the lowest index;
//   k_col_last     finishes the block's last column.
// Other V, two launches per column:
//   k_col_assign   the direct form in float32 on the vector units, merged the
//                  same way;
//   k_col_finalize reads the winners, writes indices, What and E, clears the
//                  other key buffer for the next column, and applies the
//                  in-block update to the rows j of the block (a 2D grid over
//                  elements and groups of rows).
// Per block: k_block_gemm, Wt[s+B:, :] -= U[s:s+B, s+B:]^T Et[s:s+B, :], a
// float32 matrix-core GEMM (v_mfma_f32_32x32x2f32) over double-buffered LDS
// panels.
#include "vq_internal.h"

namespace vq {
namespace {

constexpr int kTr = 32;             // transpose tile
constexpr int kAsgThreads = 256;
constexpr int kAsgChunk = 256;      // centroids per assignment workgroup
constexpr int kFinThreads = 256;
constexpr int kFinRows = 16;        // in-block rows per finalize workgroup

// dst [Cc x R] = src [R x Cc]^T through a padded LDS tile.
__global__ __launch_bounds__(256) void k_transpose(const float* __restrict__ src, int64_t R, int64_t Cc,
                                                   float* __restrict__ dst)
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
        if (r < R && c < Cc) dst[c * R + r] = t[tx][k];
    }
}

__global__ void k_fill_u64(unsigned long long* __restrict__ p, int64_t n, unsigned long long v)
{
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q < n) p[q] = v;
}

// Nearest codebook row of each sub-vector of x (one column, nv sub-vectors of
// V floats, any V) among the workgroup's chunk of centroids, direct form in
// float32 on the vector units; the chunk's winner is merged into keys[v] as
// (order-preserving bits of the distance, index).
__device__ inline unsigned sortable(float f)
{
    const unsigned u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kAsgThreads) void k_col_assign(const float* __restrict__ x, int nv, int V,
                                                            const float* __restrict__ C, int K,
                                                            unsigned long long* __restrict__ keys)
{
    __shared__ float cs[kAsgChunk * 8];
    const int k0 = blockIdx.y * kAsgChunk;
    const int kn = K - k0 < kAsgChunk ? K - k0 : kAsgChunk;
    for (int q = threadIdx.x; q < kn * V; q += kAsgThreads) cs[q] = C[(size_t)k0 * V + q];
    __syncthreads();
    const int v = blockIdx.x * kAsgThreads + threadIdx.x;
    if (v >= nv) return;
    float xv[8];
    for (int t = 0; t < 8; ++t) xv[t] = t < V ? x[(size_t)v * V + t] : 0.0f;
    float best = __builtin_inff();
    int arg = 0;
    for (int k = 0; k < kn; ++k) {
        float dist = 0.0f;
        for (int t = 0; t < V; ++t) {
            const float df = xv[t] - cs[k * V + t];
            dist = fmaf(df, df, dist);
        }
        if (dist < best) { best = dist; arg = k; }
    }
    const unsigned long long key = ((unsigned long long)sortable(best) << 32) | (unsigned)(k0 + arg);
    atomicMin(&keys[v], key);
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
// and its four wavefronts search them for 32 sub-vectors each; the chunk's
// winner enters one of kKeySlots copies of keys[v] as (order-preserving bits
// of -acc, index) through atomicMin; readers take the smallest copy.  Scores
// of different chunks are comparable: the wave grouping of sub-vectors, hence
// sx, is the same in every chunk.
constexpr int kVpChunk = 512;        // centroids per workgroup (prepared codebook is padded to whole chunks)
constexpr int kHnShift = 9;          // hn 2^(2 sc) < 2^22, its pieces below 2^13

constexpr int kKeySlots = 4;         // key copies per column: chunk y merges into slot y % kKeySlots

// Key buffers of the V = 8 path: three columns in rotation, each with
// kKeySlots copies of nv keys (spreading the atomicMin traffic of the
// K-chunk workgroups over several addresses); a column's winner is the
// smallest key over its slots.
__device__ inline size_t key_at(int nv, int slot, int64_t n, int j)
{
    return ((size_t)(n % 3) * kKeySlots + (size_t)slot) * (size_t)nv + (size_t)j;
}

__device__ inline unsigned long long key_min(const unsigned long long* __restrict__ keys, int nv, int64_t n, int j)
{
    unsigned long long k = ~0ull;
#pragma unroll
    for (int q = 0; q < kKeySlots; ++q) {
        const unsigned long long o = keys[key_at(nv, q, n, j)];
        k = o < k ? o : k;
    }
    return k;
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

__global__ __launch_bounds__(256) void k_col_step_h16(
    float* __restrict__ Wt, int64_t M, int nv, int64_t n, int64_t s, int64_t s_end, const float* __restrict__ C,
    const float* __restrict__ U, int64_t N, unsigned long long* __restrict__ keys, float* __restrict__ Xc,
    uint16_t* __restrict__ idx, float* __restrict__ Wht, float* __restrict__ Et, const vp_h16x8* __restrict__ Phi,
    const vp_h16x8* __restrict__ Plo, const vp_h16x8* __restrict__ Phn, const float* __restrict__ cmax, int K)
{
    __shared__ vp_h16x8 L[3][kVpChunk];
    const int k0 = blockIdx.y * kVpChunk;
    const int kn = K - k0 < kVpChunk ? K - k0 : kVpChunk;
    for (int q = threadIdx.x; q < kVpChunk; q += 256) {
        L[0][q] = Phi[k0 + q];
        L[1][q] = Plo[k0 + q];
        L[2][q] = Phn[k0 + q];
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j0 = (blockIdx.x * 4 + wave) * 32;
    const int jl = lane & 31, half = lane >> 5;
    const int j = j0 + jl;
    float xv[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) xv[t] = 0.0f;
    if (j < nv) {
        const float4* w4 = reinterpret_cast<const float4*>(Wt + n * M) + 2 * (size_t)j;
        const float4 wa = w4[0], wb = w4[1];
        const float w[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
        if (n > s) {
            // column n-1 of the block: its winner, value, error; the error's
            // share of column n is applied here (every workgroup of these rows
            // forms the same values), its share of the block's later columns
            // is split over the workgroups of these rows by column
            const int64_t p = n - 1;
            const unsigned kp = (unsigned)(key_min(keys, nv, p, j) & 0xFFFFFFFFull);
            const float4* c4 = reinterpret_cast<const float4*>(C) + 2 * (size_t)kp;
            const float4 ca = c4[0], cb = c4[1];
            const float qv[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
            const float* xp = Xc + (size_t)(p & 1) * M + (size_t)j * 8;
            const float unn = U[p * N + p], un = U[p * N + n];
            float e[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                e[t] = (xp[t] - qv[t]) / unn;
                xv[t] = fmaf(-e[t], un, w[t]);
            }
            if (blockIdx.y == 0 && half == 0) {
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    Wht[p * M + (int64_t)j * 8 + t] = qv[t];
                    Et[p * M + (int64_t)j * 8 + t] = e[t];
                }
                idx[p * nv + j] = (uint16_t)kp;
            }
            for (int64_t r = n + 1 + blockIdx.y; r < s_end; r += gridDim.y) {
                const float u = U[p * N + r];
                float* wr = Wt + r * M + (int64_t)j * 8 + half * 4;
#pragma unroll
                for (int t = 0; t < 4; ++t) wr[t] = fmaf(-e[half * 4 + t], u, wr[t]);
            }
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) xv[t] = w[t];
        }
        if (blockIdx.y == 0 && half == 0) {
#pragma unroll
            for (int t = 0; t < 8; ++t) Xc[(size_t)(n & 1) * M + (size_t)j * 8 + t] = xv[t];
#pragma unroll
            for (int q = 0; q < kKeySlots; ++q) keys[key_at(nv, q, n + 1, j)] = ~0ull;
        }
    }
    __syncthreads();
    if (j0 >= nv) return;
    // the wave's scale (both halves hold the same 32 sub-vectors)
    float mx = 0.0f;
#pragma unroll
    for (int t = 0; t < 8; ++t) mx = fmaxf(mx, fabsf(xv[t]));
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const int sc = vp_scale_exp(*cmax);
    const int sx = min(vp_scale_exp(mx), sc + 15 - kHnShift);
    const int eb = kHnShift + sx - sc;                  // <= 15: b is a finite fp16
    const _Float16 b = eb >= -24 ? (_Float16)(-ldexpf(1.0f, eb)) : (_Float16)0.0f;
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
    float best = -__builtin_inff();
    int bi = 0;
    const int ntiles = (kn + 31) / 32;
    auto scan = [&](vp_f32x16 acc, int tb) {
        if (tb + 32 > kn) {                              // the chunk's last, partial tile
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (tb + (r >> 2) * 8 + half * 4 + (r & 3) >= kn) acc[r] = -__builtin_inff();
        }
        float m = acc[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) m = fmaxf(m, acc[r]);
        if (m > best) {
            int rr = 0;
#pragma unroll
            for (int r = 15; r >= 0; --r)
                if (acc[r] == m) rr = r;
            best = m;
            bi = tb + (rr >> 2) * 8 + half * 4 + (rr & 3);
        }
    };
    const vp_f32x16 zero = {};
    int tb = 0;
    for (; tb + 32 < ntiles * 32; tb += 64) {
        vp_f32x16 a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A1[tb + jl], bh, zero, 0, 0, 0);
        vp_f32x16 a1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A1[tb + 32 + jl], bh, zero, 0, 0, 0);
        a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A2[tb + jl], b2, a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A2[tb + 32 + jl], b2, a1, 0, 0, 0);
        scan(a0, tb);
        scan(a1, tb + 32);
    }
    if (tb < ntiles * 32) {
        vp_f32x16 a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A1[tb + jl], bh, zero, 0, 0, 0);
        a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A2[tb + jl], b2, a0, 0, 0, 0);
        scan(a0, tb);
    }
    const float sco = -best + 0.0f;                      // -0 -> +0: one key per score
    unsigned long long key = ((unsigned long long)sortable(sco) << 32) | (unsigned)(k0 + bi);
    const unsigned long long other = __shfl_xor(key, 32);
    key = other < key ? other : key;
    if (half == 0 && j < nv) atomicMin(&keys[key_at(nv, blockIdx.y % kKeySlots, n, j)], key);
}

// The block's last column n (V = 8 path): winner, value and error; nothing of
// the block is left to update.
__global__ __launch_bounds__(256) void k_col_last(int64_t M, int nv, int64_t n, const float* __restrict__ C,
                                                  const float* __restrict__ U, int64_t N,
                                                  const unsigned long long* __restrict__ keys,
                                                  const float* __restrict__ Xc, uint16_t* __restrict__ idx,
                                                  float* __restrict__ Wht, float* __restrict__ Et)
{
    const int64_t m = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (m >= M) return;
    const int v = (int)(m >> 3), t = (int)(m & 7);
    const unsigned k = (unsigned)(key_min(keys, nv, n, v) & 0xFFFFFFFFull);
    const float wq = C[(size_t)k * 8 + t];
    const float e = (Xc[(size_t)(n & 1) * M + m] - wq) / U[n * N + n];
    Wht[n * M + m] = wq;
    Et[n * M + m] = e;
    if (t == 0) idx[n * nv + v] = (uint16_t)k;
}

// Column n: winners -> indices, What, E; the other key buffer is cleared for
// the next column; the block's rows j in (n, s_end) receive -E[:,n] U[n,j].
// Grid: x over the M elements, y over groups of kFinRows rows.
__global__ __launch_bounds__(kFinThreads) void k_col_finalize(
    float* __restrict__ Wt, int64_t M, int V, int nv, int64_t n, int64_t s_end, const float* __restrict__ C,
    const float* __restrict__ U, int64_t N, const unsigned long long* __restrict__ keys,
    unsigned long long* __restrict__ keys_next, uint16_t* __restrict__ idx, float* __restrict__ Wht,
    float* __restrict__ Et)
{
    const int64_t m = (int64_t)blockIdx.x * kFinThreads + threadIdx.x;
    if (m >= M) return;
    const int v = (int)(m / V);
    const int t = (int)(m - (int64_t)v * V);
    const unsigned k = (unsigned)(keys[v] & 0xFFFFFFFFull);
    const float wq = C[(size_t)k * V + t];
    const float e = (Wt[n * M + m] - wq) / U[n * N + n];
    const int64_t j0 = n + 1 + (int64_t)blockIdx.y * kFinRows;
    const int64_t j1 = j0 + kFinRows < s_end ? j0 + kFinRows : s_end;
    for (int64_t j = j0; j < j1; ++j) Wt[j * M + m] = fmaf(-e, U[n * N + j], Wt[j * M + m]);
    if (blockIdx.y == 0) {
        Wht[n * M + m] = wq;
        Et[n * M + m] = e;
        if (t == 0) {
            idx[n * nv + v] = (uint16_t)k;
            keys_next[v] = ~0ull;
        }
    }
}

// Wt[s_end + r, m] -= sum_k U[s + k, s_end + r] * Et[s + k, m], k < kb, for a
// 128 x 128 tile of (r, m).  k runs in chunks of kGemmK through double-buffered
// LDS panels (k the slow index; the next chunk is loaded into registers while
// the current one is used, one barrier per chunk).  Each of the 8 wavefronts
// accumulates a 32 x 64 block as two 32 x 32 blocks of v_mfma_f32_32x32x2f32
// (lane l feeds A[l%32][l/32] and B[l/32][l%32]); k pairs are taken in
// increasing order.
constexpr int kGemmT = 128;          // output tile edge
constexpr int kGemmK = 16;           // k per LDS chunk
constexpr int kGemmLd = kGemmT + 4;  // padded LDS row

__global__ __launch_bounds__(512) void k_block_gemm(float* __restrict__ Wt, const float* __restrict__ U,
                                                    const float* __restrict__ Et, int64_t N, int64_t M,
                                                    int64_t s, int kb, int64_t s_end)
{
    __shared__ float As[2][kGemmK][kGemmLd];
    __shared__ float Bs[2][kGemmK][kGemmLd];
    const int64_t R = N - s_end;
    const int64_t r0 = (int64_t)blockIdx.y * kGemmT, m0 = (int64_t)blockIdx.x * kGemmT;
    const int tid = threadIdx.x;
    // loader: thread -> (k = tid / 32, columns 4 * (tid % 32) .. + 4) of each panel
    const int lk_ = tid >> 5, lc = (tid & 31) * 4;
    float ra[4], rb[4];
    auto load = [&](int kc) {
        const int k = kc + lk_;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = r0 + lc + i, mm = m0 + lc + i;
            ra[i] = (k < kb && r < R) ? U[(s + k) * N + s_end + r] : 0.0f;
            rb[i] = (k < kb && mm < M) ? Et[(s + k) * M + mm] : 0.0f;
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            As[buf][lk_][lc + i] = ra[i];
            Bs[buf][lk_][lc + i] = rb[i];
        }
    };
    const int lane = tid & 63, wave = tid >> 6;
    const int wr = (wave & 3) * 32, wc = (wave >> 2) * 64;
    const int li = lane & 31, lk = lane >> 5;
    typedef float f16x_t __attribute__((ext_vector_type(16)));
    f16x_t acc0, acc1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { acc0[r] = 0.0f; acc1[r] = 0.0f; }
    const int nk = (kb + kGemmK - 1) / kGemmK;
    load(0);
    store(0);
    __syncthreads();
    for (int c = 0; c < nk; ++c) {
        const int buf = c & 1;
        if (c + 1 < nk) load((c + 1) * kGemmK);
#pragma unroll
        for (int kk = 0; kk < kGemmK; kk += 2) {
            const float a = As[buf][kk + lk][wr + li];
            const float b0 = Bs[buf][kk + lk][wc + li];
            const float b1 = Bs[buf][kk + lk][wc + 32 + li];
            acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b0, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b1, acc1, 0, 0, 0);
        }
        if (c + 1 < nk) store(buf ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t mm = m0 + wc + h * 32 + li;
        if (mm >= M) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = r0 + wr + (r >> 2) * 8 + lk * 4 + (r & 3);
            if (row < R) {
                float* p = Wt + (s_end + row) * M + mm;
                *p = *p - (h ? acc1[r] : acc0[r]);
            }
        }
    }
}

}  // namespace

size_t ws_vptq(int64_t M, int64_t N, int V)
{
    const int64_t nv = M / V;
    // three transposed M x N copies, three key buffers (kKeySlots slots each), two working columns,
    // the prepared codebook (3 x 16 bytes per centroid, at most 65536), max |C|
    return 3 * align_up((size_t)M * (size_t)N * sizeof(float)) + align_up((size_t)(3 * kKeySlots * nv) * sizeof(uint64_t)) +
           align_up((size_t)(2 * M) * sizeof(float)) + 3 * align_up((size_t)65536 * sizeof(vp_h16x8)) +
           align_up(sizeof(float));
}

vq_status vptq_launch(const float* W, const float* U, int64_t M, int64_t N, int V, const float* C, int K, int B,
                      uint16_t* idx, float* W_hat, float* E, void* ws, size_t ws_bytes, hipStream_t st)
{
    const int64_t nv = M / V;
    Carver cv(ws, ws_bytes);
    float* Wt = cv.take<float>((size_t)(M * N));
    float* Wht = cv.take<float>((size_t)(M * N));
    float* Et = cv.take<float>((size_t)(M * N));
    unsigned long long* keys = cv.take<unsigned long long>((size_t)(3 * kKeySlots * nv));
    float* Xc = cv.take<float>((size_t)(2 * M));
    const int Kp = (K + kVpChunk - 1) / kVpChunk * kVpChunk;
    vp_h16x8* Phi = cv.take<vp_h16x8>(65536);
    vp_h16x8* Plo = cv.take<vp_h16x8>(65536);
    vp_h16x8* Phn = cv.take<vp_h16x8>(65536);
    float* cmax = cv.take<float>(1);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_vptq: workspace too small");
    TimedRegion tr("vptq", K, st);
    const dim3 tw(grid_for(N, kTr), grid_for(M, kTr));
    hipLaunchKernelGGL(k_transpose, tw, dim3(256), 0, st, W, M, N, Wt);
    VQ_LAUNCHED("k_transpose");
    hipLaunchKernelGGL(k_fill_u64, dim3(grid_for(3 * kKeySlots * nv, 256)), dim3(256), 0, st, keys,
                       3 * kKeySlots * nv, ~0ull);
    VQ_LAUNCHED("k_fill_u64");
    const bool v8 = V == 8 && aligned16(C) && (M % 4 == 0);
    if (v8) {
        hipLaunchKernelGGL(k_vp_absmax, dim3(1), dim3(1024), 0, st, reinterpret_cast<const float4*>(C),
                           (int64_t)K * 2, cmax);
        VQ_LAUNCHED("k_vp_absmax");
        hipLaunchKernelGGL(k_vp_prep, dim3(grid_for(Kp, 256)), dim3(256), 0, st, C, K, Kp, cmax, Phi, Plo, Phn);
        VQ_LAUNCHED("k_vp_prep");
    }
    const dim3 ga(grid_for(nv, kAsgThreads), grid_for(K, kAsgChunk));
    const dim3 gm(grid_for(nv, 128), (unsigned)(Kp / kVpChunk));
    for (int64_t s = 0; s < N; s += B) {
        const int64_t s_end = s + B < N ? s + B : N;
        if (v8) {
            // one launch per column (it also finishes the column before it),
            // and one for the block's last column
            for (int64_t n = s; n < s_end; ++n) {
                hipLaunchKernelGGL(k_col_step_h16, gm, dim3(256), 0, st, Wt, M, (int)nv, n, s, s_end, C, U, N, keys,
                                   Xc, idx, Wht, Et, Phi, Plo, Phn, cmax, K);
                VQ_LAUNCHED("k_col_step_h16");
            }
            hipLaunchKernelGGL(k_col_last, dim3(grid_for(M, 256)), dim3(256), 0, st, M, (int)nv, s_end - 1, C, U, N,
                               keys, Xc, idx, Wht, Et);
            VQ_LAUNCHED("k_col_last");
        } else {
            for (int64_t n = s; n < s_end; ++n) {
                unsigned long long* kc = (n & 1) ? keys + nv : keys;
                unsigned long long* kn = (n & 1) ? keys : keys + nv;
                hipLaunchKernelGGL(k_col_assign, ga, dim3(kAsgThreads), 0, st, Wt + n * M, (int)nv, V, C, K, kc);
                VQ_LAUNCHED("k_col_assign");
                const int64_t rows = s_end - n - 1;
                const dim3 gf(grid_for(M, kFinThreads),
                              (unsigned)(rows > 0 ? (rows + kFinRows - 1) / kFinRows : 1));
                hipLaunchKernelGGL(k_col_finalize, gf, dim3(kFinThreads), 0, st, Wt, M, V, (int)nv, n, s_end, C, U,
                                   N, kc, kn, idx, Wht, Et);
                VQ_LAUNCHED("k_col_finalize");
            }
        }
        if (s_end < N) {
            TimedRegion tg("vptq_block_update", K, st);
            const dim3 gg(grid_for(M, kGemmT), grid_for(N - s_end, kGemmT));
            hipLaunchKernelGGL(k_block_gemm, gg, dim3(512), 0, st, Wt, U, Et, N, M, s, (int)(s_end - s), s_end);
            VQ_LAUNCHED("k_block_gemm");
        }
    }
    const dim3 tb(grid_for(M, kTr), grid_for(N, kTr));
    hipLaunchKernelGGL(k_transpose, tb, dim3(256), 0, st, Wht, N, M, W_hat);
    VQ_LAUNCHED("k_transpose");
    if (E) {
        hipLaunchKernelGGL(k_transpose, tb, dim3(256), 0, st, Et, N, M, E);
        VQ_LAUNCHED("k_transpose");
    }
    return VQ_OK;
}

}  // namespace vq
