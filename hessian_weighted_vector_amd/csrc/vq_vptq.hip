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
// Per column, two launches:
//   k_col_assign   the M/V x K distances of the column; V = 8 on the float32
//                  matrix cores (k_col_assign_mfma, expanded form), other V
//                  in the direct form on the vector units; workgroups split K,
//                  each stages its centroids in LDS, and the per-sub-vector
//                  minima meet in a packed 64-bit atomicMin of (score bits,
//                  index): the order of arrival does not matter, and equal
//                  scores keep the lowest index;
//   k_col_finalize reads the winners, writes indices, What and E, clears the
//                  other key buffer for the next column, and applies the
//                  in-block update to the rows j of the block (a 2D grid over
//                  elements and groups of rows).
// Per block: k_block_gemm, Wt[s+B:, :] -= U[s:s+B, s+B:]^T Et[s:s+B, :], a
// float32 matrix-core GEMM (v_mfma_f32_32x32x2f32) over LDS panels.
#include "vq_internal.h"

namespace vq {
namespace {

constexpr int kTr = 32;             // transpose tile
constexpr int kAsgThreads = 256;
constexpr int kAsgChunk = 256;      // centroids per assignment workgroup
constexpr int kFinThreads = 256;
constexpr int kFinRows = 16;        // in-block rows per finalize workgroup
constexpr int kGemmTile = 64;       // output tile of the block update
constexpr int kGemmMaxK = 128;      // largest block size the GEMM stages at once

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

// V = 8 on the float32 matrix cores.  ||x - c||^2 = ||x||^2 + 2 (||c||^2 / 2
// - <c, x>): the workgroup stages kMChunk centroids transposed in LDS (k
// slow, so the 32 lanes that feed one MFMA row read consecutive words) with
// their half norms; each wavefront takes 32 sub-vectors and, per tile of 32
// centroids, forms the 32 x 32 inner products with four
// v_mfma_f32_32x32x2f32 (lane l feeds A = c_{l%32}[2s + l/32] and
// B = x_{l%32}[2s + l/32]) and scans its 16 accumulator rows (centroid
// (r/4)*8 + (l/32)*4 + r%4 of the tile) in increasing index order.  The two
// lanes holding one sub-vector merge, then the chunk's winner enters keys[v]
// as (order-preserving bits of the score, index) through atomicMin.
constexpr int kMChunk = 256;

__global__ __launch_bounds__(256) void k_col_assign_mfma(const float* __restrict__ x, int nv,
                                                         const float* __restrict__ C, int K,
                                                         unsigned long long* __restrict__ keys)
{
    __shared__ float csT[8][kMChunk];
    __shared__ float hn[kMChunk];
    const int k0 = blockIdx.y * kMChunk;
    const int kn = K - k0 < kMChunk ? K - k0 : kMChunk;
    for (int q = threadIdx.x; q < kMChunk; q += 256) {
        float c[8];
        if (q < kn) {
            const float4 a = reinterpret_cast<const float4*>(C)[2 * (size_t)(k0 + q)];
            const float4 b = reinterpret_cast<const float4*>(C)[2 * (size_t)(k0 + q) + 1];
            c[0] = a.x; c[1] = a.y; c[2] = a.z; c[3] = a.w; c[4] = b.x; c[5] = b.y; c[6] = b.z; c[7] = b.w;
            float nrm = 0.0f;
#pragma unroll
            for (int t = 0; t < 8; ++t) nrm = fmaf(c[t], c[t], nrm);
            hn[q] = 0.5f * nrm;
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) c[t] = 0.0f;
            hn[q] = __builtin_inff();   // padding never wins
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) csT[t][q] = c[t];
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j0 = (blockIdx.x * 4 + wave) * 32;
    if (j0 >= nv) return;
    const int jl = lane & 31, half = lane >> 5;
    const int j = j0 + jl;
    float xb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) xb[s] = j < nv ? x[(size_t)j * 8 + 2 * s + half] : 0.0f;
    typedef float f16x_t __attribute__((ext_vector_type(16)));
    float best = __builtin_inff();
    int bi = 0;
    const int ntiles = (kn + 31) / 32;
    // The tile's minimum first; the row is located only when it beats the
    // running best (rare after the first tiles), scanning rows in increasing
    // index order so equal scores keep the lowest index.  Two tiles per step
    // keep two independent MFMA chains in flight.
    auto scan = [&](const f16x_t& acc, int tb) {
        float sc[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[r] = hn[tb + (r >> 2) * 8 + half * 4 + (r & 3)] - acc[r];
        float m = sc[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) m = fminf(m, sc[r]);
        if (m < best) {
            int rr = 0;
#pragma unroll
            for (int r = 15; r >= 0; --r)
                if (sc[r] == m) rr = r;
            best = m;
            bi = tb + (rr >> 2) * 8 + half * 4 + (rr & 3);
        }
    };
    int tb = 0;
    for (; tb + 32 < ntiles * 32; tb += 64) {
        f16x_t a0, a1;
#pragma unroll
        for (int r = 0; r < 16; ++r) { a0[r] = 0.0f; a1[r] = 0.0f; }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            a0 = __builtin_amdgcn_mfma_f32_32x32x2f32(csT[2 * s + half][tb + jl], xb[s], a0, 0, 0, 0);
            a1 = __builtin_amdgcn_mfma_f32_32x32x2f32(csT[2 * s + half][tb + 32 + jl], xb[s], a1, 0, 0, 0);
        }
        scan(a0, tb);
        scan(a1, tb + 32);
    }
    if (tb < ntiles * 32) {
        f16x_t a0;
#pragma unroll
        for (int r = 0; r < 16; ++r) a0[r] = 0.0f;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            a0 = __builtin_amdgcn_mfma_f32_32x32x2f32(csT[2 * s + half][tb + jl], xb[s], a0, 0, 0, 0);
        scan(a0, tb);
    }
    unsigned long long key = ((unsigned long long)sortable(best) << 32) | (unsigned)(k0 + bi);
    const unsigned long long other = __shfl_xor(key, 32);
    key = other < key ? other : key;
    if (half == 0 && j < nv) atomicMin(&keys[j], key);
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
// 64 x 64 tile of (r, m).  The U and Et panels of the tile sit in LDS with k
// as the slow index; each of the 4 wavefronts accumulates one 32 x 32 block
// with v_mfma_f32_32x32x2f32 (lane l feeds A[l%32][l/32] and B[l/32][l%32]).
__global__ __launch_bounds__(256) void k_block_gemm(float* __restrict__ Wt, const float* __restrict__ U,
                                                    const float* __restrict__ Et, int64_t N, int64_t M,
                                                    int64_t s, int kb, int64_t s_end)
{
    __shared__ float As[kGemmMaxK][kGemmTile];
    __shared__ float Bs[kGemmMaxK][kGemmTile];
    const int64_t R = N - s_end;
    const int64_t r0 = (int64_t)blockIdx.y * kGemmTile, m0 = (int64_t)blockIdx.x * kGemmTile;
    const int kp = (kb + 1) & ~1;   // padded to the MFMA's k of 2
    for (int q = threadIdx.x; q < kp * kGemmTile; q += 256) {
        const int k = q / kGemmTile, c = q - k * kGemmTile;
        const int64_t r = r0 + c, mm = m0 + c;
        As[k][c] = (k < kb && r < R) ? U[(s + k) * N + s_end + r] : 0.0f;
        Bs[k][c] = (k < kb && mm < M) ? Et[(s + k) * M + mm] : 0.0f;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;
    const int li = lane & 31, lk = lane >> 5;
    typedef float f16x_t __attribute__((ext_vector_type(16)));
    f16x_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    for (int k = 0; k < kp; k += 2) {
        const float a = As[k + lk][wr + li];
        const float b = Bs[k + lk][wc + li];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    const int64_t mm = m0 + wc + li;
    if (mm >= M) return;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t row = r0 + wr + (r >> 2) * 8 + lk * 4 + (r & 3);
        if (row < R) {
            float* p = Wt + (s_end + row) * M + mm;
            *p = *p - acc[r];
        }
    }
}

}  // namespace

size_t ws_vptq(int64_t M, int64_t N, int V)
{
    const int64_t nv = M / V;
    return 3 * align_up((size_t)M * (size_t)N * sizeof(float)) + 2 * align_up((size_t)nv * sizeof(uint64_t));
}

vq_status vptq_launch(const float* W, const float* U, int64_t M, int64_t N, int V, const float* C, int K, int B,
                      uint16_t* idx, float* W_hat, float* E, void* ws, size_t ws_bytes, hipStream_t st)
{
    const int64_t nv = M / V;
    Carver cv(ws, ws_bytes);
    float* Wt = cv.take<float>((size_t)(M * N));
    float* Wht = cv.take<float>((size_t)(M * N));
    float* Et = cv.take<float>((size_t)(M * N));
    unsigned long long* keys0 = cv.take<unsigned long long>((size_t)nv);
    unsigned long long* keys1 = cv.take<unsigned long long>((size_t)nv);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_vptq: workspace too small");
    TimedRegion tr("vptq", K, st);
    const dim3 tw(grid_for(N, kTr), grid_for(M, kTr));
    hipLaunchKernelGGL(k_transpose, tw, dim3(256), 0, st, W, M, N, Wt);
    VQ_LAUNCHED("k_transpose");
    hipLaunchKernelGGL(k_fill_u64, dim3(grid_for(nv, 256)), dim3(256), 0, st, keys0, nv, ~0ull);
    VQ_LAUNCHED("k_fill_u64");
    hipLaunchKernelGGL(k_fill_u64, dim3(grid_for(nv, 256)), dim3(256), 0, st, keys1, nv, ~0ull);
    VQ_LAUNCHED("k_fill_u64");
    const bool v8 = V == 8 && aligned16(C) && (M % 4 == 0);
    const dim3 ga(grid_for(nv, kAsgThreads), grid_for(K, kAsgChunk));
    const dim3 gm(grid_for(nv, 128), grid_for(K, kMChunk));
    for (int64_t s = 0; s < N; s += B) {
        const int64_t s_end = s + B < N ? s + B : N;
        for (int64_t n = s; n < s_end; ++n) {
            unsigned long long* kc = (n & 1) ? keys1 : keys0;
            unsigned long long* kn = (n & 1) ? keys0 : keys1;
            if (v8)
                hipLaunchKernelGGL(k_col_assign_mfma, gm, dim3(256), 0, st, Wt + n * M, (int)nv, C, K, kc);
            else
                hipLaunchKernelGGL(k_col_assign, ga, dim3(kAsgThreads), 0, st, Wt + n * M, (int)nv, V, C, K, kc);
            VQ_LAUNCHED("k_col_assign");
            const int64_t rows = s_end - n - 1;
            const dim3 gf(grid_for(M, kFinThreads), (unsigned)(rows > 0 ? (rows + kFinRows - 1) / kFinRows : 1));
            hipLaunchKernelGGL(k_col_finalize, gf, dim3(kFinThreads), 0, st, Wt, M, V, (int)nv, n, s_end, C, U, N,
                               kc, kn, idx, Wht, Et);
            VQ_LAUNCHED("k_col_finalize");
        }
        if (s_end < N) {
            TimedRegion tg("vptq_block_update", K, st);
            const dim3 gg(grid_for(M, kGemmTile), grid_for(N - s_end, kGemmTile));
            hipLaunchKernelGGL(k_block_gemm, gg, dim3(256), 0, st, Wt, U, Et, N, M, s, (int)(s_end - s), s_end);
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
