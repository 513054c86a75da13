// Bandwidth-bound passes: bi-normalization, residual, reconstruction and the
// objective.  Every float64 reduction here runs in a fixed order (per-thread
// strided sums, then a fixed tree), so results are bitwise reproducible.
#include "vq_internal.h"

namespace vq {
namespace {

constexpr int kBlock = 256;

// Streaming accesses of the residual pass: the nontemporal hint lets the
// matrix stream pass through L2 without evicting the codebook that every
// sub-vector gathers from.
typedef float vf4_t __attribute__((ext_vector_type(4)));
__device__ inline float4 ld_stream(const float4* p)
{
    const vf4_t v = __builtin_nontemporal_load(reinterpret_cast<const vf4_t*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ inline void st_stream(float4* p, float4 v)
{
    vf4_t w;
    w.x = v.x; w.y = v.y; w.z = v.z; w.w = v.w;
    __builtin_nontemporal_store(w, reinterpret_cast<vf4_t*>(p));
}
__device__ inline int ld_stream(const uint16_t* p) { return __builtin_nontemporal_load(p); }

// Fixed-order tree reduction of one double per thread (blockDim == 256).
__device__ inline double block_sum_f64(double v, double* sh)
{
    sh[threadIdx.x] = v;
    __syncthreads();
    for (int w = kBlock / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) sh[threadIdx.x] = sh[threadIdx.x] + sh[threadIdx.x + w];
        __syncthreads();
    }
    double r = sh[0];
    __syncthreads();
    return r;
}

// ---- bi-normalization (SCVQ summary: rows and columns bi-normalized) ----
// r_i = sqrt(sum_j W_ij^2 / N) in float64, 1 when zero; rho_i = r_i^2.
__global__ __launch_bounds__(kBlock) void k_row_rms(const float* __restrict__ W, int64_t N,
                                                    float* __restrict__ r, float* __restrict__ rho)
{
    __shared__ double sh[kBlock];
    const int64_t i = blockIdx.x;
    const float* row = W + i * N;
    double acc = 0.0;
    for (int64_t j = threadIdx.x; j < N; j += kBlock) {
        const double w = (double)row[j];
        acc = acc + w * w;
    }
    const double tot = block_sum_f64(acc, sh);
    if (threadIdx.x == 0) {
        float ri = (float)sqrt(tot / (double)N);
        if (ri == 0.0f) ri = 1.0f;
        r[i] = ri;
        const double rd = (double)ri;
        rho[i] = (float)(rd * rd);
    }
}

// Partial column sums of (W_ij / r_i)^2 over one group of rows.
// Block = 64 columns x 4 row lanes; grid = (column chunks, row groups).
__global__ __launch_bounds__(kBlock) void k_col_partial(const float* __restrict__ W,
                                                        const float* __restrict__ r, int64_t M,
                                                        int64_t N, int64_t rows_per_group,
                                                        double* __restrict__ part)
{
    __shared__ double sh[4][64];
    const int cl = threadIdx.x & 63;
    const int rl = threadIdx.x >> 6;
    const int64_t j = (int64_t)blockIdx.x * 64 + cl;
    const int64_t i0 = (int64_t)blockIdx.y * rows_per_group;
    const int64_t i1 = i0 + rows_per_group < M ? i0 + rows_per_group : M;
    double acc = 0.0;
    if (j < N) {
        for (int64_t i = i0 + rl; i < i1; i += 4) {
            const float wt = W[i * N + j] / r[i];
            const double w = (double)wt;
            acc = acc + w * w;
        }
    }
    sh[rl][cl] = acc;
    __syncthreads();
    if (rl == 0 && j < N) {
        const double tot = ((sh[0][cl] + sh[1][cl]) + sh[2][cl]) + sh[3][cl];
        part[(int64_t)blockIdx.y * N + j] = tot;
    }
}

// c_j = sqrt(sum over row groups / M) (groups added in order), 1 when zero;
// hcol_j = h_j c_j^2 in float64.
__global__ void k_col_finish(const double* __restrict__ part, int groups, int64_t M, int64_t N,
                             const float* __restrict__ h, float* __restrict__ c,
                             float* __restrict__ hcol)
{
    const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= N) return;
    double tot = 0.0;
    for (int g = 0; g < groups; ++g) tot = tot + part[(int64_t)g * N + j];
    float cj = (float)sqrt(tot / (double)M);
    if (cj == 0.0f) cj = 1.0f;
    c[j] = cj;
    const double cd = (double)cj;
    hcol[j] = (float)((double)h[j] * cd * cd);
}

// W'_ij = (W_ij / r_i) / c_j in float32.
__global__ void k_binorm_apply(const float* __restrict__ W, const float* __restrict__ r,
                               const float* __restrict__ c, int64_t M, int64_t N,
                               float* __restrict__ Wp)
{
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= M * N) return;
    const int64_t i = e / N;
    const int64_t j = e - i * N;
    const float wt = W[e] / r[i];
    Wp[e] = wt / c[j];
}

// ---- residual (VPTQ page, "Residual Vector Quantization") ---------------
// An index >= K (a caller error) yields NaN instead of an out-of-range read.
__global__ void k_residual(const float* __restrict__ X, int64_t total, int d,
                           const float* __restrict__ C, int K, const uint16_t* __restrict__ idx,
                           float* __restrict__ R)
{
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= total) return;
    const int64_t s = e / d;
    const int t = (int)(e - s * d);
    const int k = idx[s];
    R[e] = k < K ? X[e] - C[(size_t)k * d + t] : __builtin_nanf("");
}

// d == 8 with 16-byte aligned buffers: one thread per half sub-vector.
__global__ void k_residual8(const float4* __restrict__ X, int64_t n_half, const float4* __restrict__ C, int K,
                            const uint16_t* __restrict__ idx, float4* __restrict__ R)
{
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= n_half) return;
    const int k = ld_stream(idx + (q >> 1));
    const float4 x = ld_stream(X + q);
    float4 r;
    if (k < K) {
        const float4 c = C[(size_t)k * 2 + (q & 1)];
        r.x = x.x - c.x; r.y = x.y - c.y; r.z = x.z - c.z; r.w = x.w - c.w;
    } else {
        r.x = r.y = r.z = r.w = __builtin_nanf("");
    }
    st_stream(R + q, r);
}

// ---- reconstruction ------------------------------------------------------
// One thread per sub-vector: ((C1[i1] + C2[i2]) * c_j) * r_i, float32.
// An index >= K (a caller error) decodes to NaN instead of an out-of-range read.
__global__ void k_decode(int64_t n_sub, int64_t nb, int d, const float* __restrict__ C1, int K1,
                         const uint16_t* __restrict__ idx1, const float* __restrict__ C2, int K2,
                         const uint16_t* __restrict__ idx2, const float* __restrict__ rs,
                         const float* __restrict__ cs, float* __restrict__ Wh)
{
    const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= n_sub) return;
    const int64_t i = s / nb;
    const int64_t b = s - i * nb;
    float* out = Wh + s * d;
    const int k1 = idx1[s];
    const int k2 = C2 ? idx2[s] : 0;
    if (k1 >= K1 || (C2 && k2 >= K2)) {
        for (int t = 0; t < d; ++t) out[t] = __builtin_nanf("");
        return;
    }
    const float* c1 = C1 + (size_t)k1 * d;
    const float* c2 = C2 ? C2 + (size_t)k2 * d : nullptr;
    const float ri = rs ? rs[i] : 1.0f;
    for (int t = 0; t < d; ++t) {
        float v = c1[t];
        if (c2) v = v + c2[t];
        if (cs) v = v * cs[b * d + t];
        if (rs) v = v * ri;
        out[t] = v;
    }
}

// The exact salient values overwrite their positions (HAS-VQ abstract:
// exact reconstruction of the decoupled weights).  One workgroup per row;
// its threads stride over the row's CSR entries.
// d == 8 with 16-byte aligned buffers: 16-byte loads and stores, same
// operation order as k_decode.  Workgroups are laid out by row (bpr
// workgroups per row), so the row and its scale come from the workgroup
// number.  U half sub-vectors per thread: thread t of the
// workgroup takes halves t, t + kBlock, ..., of its slice of a row, so each
// of the U steps is a coalesced pass.  All indices and column scales are
// requested first, then all U first-stage centroid halves, so U gathers are
// in flight per lane instead of one.  With C2L the residual codebook (at most
// kC2Lds centroids) is staged in LDS once per workgroup and read from there.
// Same arithmetic and operation order as k_decode8.
constexpr int kC2Lds = 512;

template <int U, bool C2L>
__global__ __launch_bounds__(kBlock) void k_decode8u(int64_t nb, unsigned bpr, const float4* __restrict__ C1, int K1,
                                                     const uint16_t* __restrict__ idx1, const float4* __restrict__ C2,
                                                     int K2, const uint16_t* __restrict__ idx2,
                                                     const float* __restrict__ rs, const float4* __restrict__ cs,
                                                     float4* __restrict__ Wh)
{
    __shared__ float4 sC2[C2L ? 2 * kC2Lds : 1];
    if (C2L) {
        for (int q = threadIdx.x; q < 2 * K2; q += kBlock) sC2[q] = C2[q];
        __syncthreads();
    }
    const int64_t i = blockIdx.x / bpr;
    const int64_t base = (int64_t)(blockIdx.x - (unsigned)i * bpr) * (kBlock * U) + threadIdx.x;
    const float ri = rs ? rs[i] : 1.0f;
    int k1[U], k2[U];
    float4 cv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t hq = base + (int64_t)u * kBlock;
        const bool ok = hq < 2 * nb;
        const int64_t s = i * nb + (hq >> 1);
        k1[u] = ok ? (int)idx1[s] : 0;
        k2[u] = (ok && C2) ? (int)idx2[s] : 0;
        if (cs && ok) cv[u] = cs[hq];
    }
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int half = (int)((base + (int64_t)u * kBlock) & 1);
        const int kk = k1[u] < K1 ? k1[u] : 0;
        v[u] = C1[(size_t)kk * 2 + half];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t hq = base + (int64_t)u * kBlock;
        if (hq >= 2 * nb) continue;
        const int half = (int)(hq & 1);
        float4 w = v[u];
        if (k1[u] >= K1 || (C2 && k2[u] >= K2)) {
            w.x = w.y = w.z = w.w = __builtin_nanf("");
        } else {
            if (C2) {
                const float4 c = C2L ? sC2[k2[u] * 2 + half] : C2[(size_t)k2[u] * 2 + half];
                w.x = w.x + c.x; w.y = w.y + c.y; w.z = w.z + c.z; w.w = w.w + c.w;
            }
            if (cs) {
                const float4 c = cv[u];
                w.x = w.x * c.x; w.y = w.y * c.y; w.z = w.z * c.z; w.w = w.w * c.w;
            }
            if (rs) {
                w.x = w.x * ri; w.y = w.y * ri; w.z = w.z * ri; w.w = w.w * ri;
            }
        }
        Wh[i * 2 * nb + hq] = w;
    }
}

__global__ __launch_bounds__(kBlock) void k_sparse_overwrite(int64_t N, const int32_t* __restrict__ row_ptr,
                                                             const int32_t* __restrict__ col,
                                                             const float* __restrict__ val, float* __restrict__ Wh)
{
    const int64_t i = blockIdx.x;
    const int64_t e1 = row_ptr[i + 1];
    for (int64_t e = row_ptr[i] + threadIdx.x; e < e1; e += kBlock) {
        const int32_t j = col[e];
        if (j >= 0 && j < N) Wh[i * N + j] = val[e];   // an out-of-range column is skipped
    }
}

// ---- objective: per-block float64 partial sums of D(s, idx[s]) ----------
// D in the direct form, float64, terms in t order.  An index >= K (a caller
// error) makes J NaN instead of reading out of range.
__device__ __forceinline__ double objective_term(const float* __restrict__ X, const float* __restrict__ hcol,
                                                 const float* __restrict__ rho, const uint8_t* __restrict__ mask,
                                                 int64_t s, uint32_t nb, int d, const float* __restrict__ C, int K,
                                                 int k, int vec)
{
    if (k >= K) return __builtin_nan("");
    const uint32_t i = (uint32_t)(s / nb);
    const uint32_t b = (uint32_t)s - i * nb;
    const unsigned mb = mask ? mask[s] : 0u;
    float x[8], c[8], h[8];
    if (vec) {   // d == 8, 16-byte aligned buffers
        const float4* x4 = reinterpret_cast<const float4*>(X + s * 8);
        const float4* c4 = reinterpret_cast<const float4*>(C + (size_t)k * 8);
        const float4* h4 = reinterpret_cast<const float4*>(hcol + (size_t)b * 8);
        const float4 xa = x4[0], xb = x4[1], ca = c4[0], cb = c4[1], ha = h4[0], hb = h4[1];
        x[0] = xa.x; x[1] = xa.y; x[2] = xa.z; x[3] = xa.w; x[4] = xb.x; x[5] = xb.y; x[6] = xb.z; x[7] = xb.w;
        c[0] = ca.x; c[1] = ca.y; c[2] = ca.z; c[3] = ca.w; c[4] = cb.x; c[5] = cb.y; c[6] = cb.z; c[7] = cb.w;
        h[0] = ha.x; h[1] = ha.y; h[2] = ha.z; h[3] = ha.w; h[4] = hb.x; h[5] = hb.y; h[6] = hb.z; h[7] = hb.w;
    } else {
        for (int t = 0; t < 8; ++t) {
            x[t] = t < d ? X[s * d + t] : 0.f;
            c[t] = t < d ? C[(size_t)k * d + t] : 0.f;
            h[t] = t < d ? hcol[(size_t)b * d + t] : 0.f;
        }
    }
    const double rr = rho ? (double)rho[i] : 1.0;
    double D = 0.0;
    for (int t = 0; t < d; ++t) {
        double w = (double)h[t];
        if (rho) w = w * rr;
        if ((mb >> t) & 1u) w = 0.0;
        const double diff = (double)x[t] - (double)c[t];
        const double sq = diff * diff;
        D = D + w * sq;
    }
    return D;
}

// Workgroup = kObjPerBlock consecutive sub-vectors, two per thread (s and
// s + kBlock, both indices read first so the two centroid gathers overlap);
// partial = the block sum of the thread sums D(s) + D(s + kBlock).
constexpr int kObjPerBlock = 2 * kBlock;
__global__ __launch_bounds__(kBlock) void k_objective_partial(
    const float* __restrict__ X, const float* __restrict__ hcol, const float* __restrict__ rho,
    const uint8_t* __restrict__ mask, int64_t n_sub, uint32_t nb, int d,
    const float* __restrict__ C, int K, const uint16_t* __restrict__ idx, int vec, double* __restrict__ part)
{
    __shared__ double sh[kBlock];
    const int64_t s0 = (int64_t)blockIdx.x * kObjPerBlock + threadIdx.x;
    const int64_t s1 = s0 + kBlock;
    const int k0 = s0 < n_sub ? (int)idx[s0] : 0;
    const int k1 = s1 < n_sub ? (int)idx[s1] : 0;
    double D0 = 0.0, D1 = 0.0;
    if (s0 < n_sub) D0 = objective_term(X, hcol, rho, mask, s0, nb, d, C, K, k0, vec);
    if (s1 < n_sub) D1 = objective_term(X, hcol, rho, mask, s1, nb, d, C, K, k1, vec);
    const double tot = block_sum_f64(D0 + D1, sh);
    if (threadIdx.x == 0) part[blockIdx.x] = tot;
}

// One block of 1024 adds the partials: strided per-thread sums (four
// independent chains, added in a fixed order), then a fixed tree.
__global__ __launch_bounds__(1024) void k_sum_partials(const double* __restrict__ part, int64_t n,
                                                       double* __restrict__ out)
{
    __shared__ double sh[1024];
    double a[4] = {0.0, 0.0, 0.0, 0.0};
    int64_t e = threadIdx.x;
    for (; e + 3 * 1024 < n; e += 4 * 1024) {
#pragma unroll
        for (int u = 0; u < 4; ++u) a[u] = a[u] + part[e + u * 1024];
    }
    for (; e < n; e += 1024) a[0] = a[0] + part[e];
    sh[threadIdx.x] = (a[0] + a[1]) + (a[2] + a[3]);
    __syncthreads();
    for (int w = 512; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) sh[threadIdx.x] = sh[threadIdx.x] + sh[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) *out = sh[0];
}

constexpr int64_t kColChunk = 64;

constexpr int64_t kRowGroups = 32;

}  // namespace

size_t ws_binorm(int64_t M, int64_t N)
{
    (void)M;
    return align_up((size_t)kRowGroups * N * sizeof(double));
}

size_t ws_objective(int64_t n_sub) { return align_up((size_t)grid_for(n_sub, kObjPerBlock) * sizeof(double)); }

vq_status binorm_launch(const float* W, const float* h, int64_t M, int64_t N, float* Wp, float* r,
                        float* c, float* hcol, float* rho, void* ws, size_t ws_bytes, hipStream_t st)
{
    Carver cv(ws, ws_bytes);
    double* part = cv.take<double>((size_t)kRowGroups * N);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_binorm: workspace too small");
    TimedRegion tr("binorm", 0, st);
    hipLaunchKernelGGL(k_row_rms, dim3((unsigned)M), dim3(kBlock), 0, st, W, N, r, rho);
    VQ_LAUNCHED("k_row_rms");
    const int64_t rpg = (M + kRowGroups - 1) / kRowGroups;
    hipLaunchKernelGGL(k_col_partial, dim3(grid_for(N, kColChunk), (unsigned)kRowGroups), dim3(kBlock),
                       0, st, W, r, M, N, rpg, part);
    VQ_LAUNCHED("k_col_partial");
    hipLaunchKernelGGL(k_col_finish, dim3(grid_for(N, kBlock)), dim3(kBlock), 0, st, part,
                       (int)kRowGroups, M, N, h, c, hcol);
    VQ_LAUNCHED("k_col_finish");
    hipLaunchKernelGGL(k_binorm_apply, dim3(grid_for(M * N, kBlock)), dim3(kBlock), 0, st, W, r, c, M,
                       N, Wp);
    VQ_LAUNCHED("k_binorm_apply");
    return VQ_OK;
}

vq_status residual_launch(const float* X, int64_t M, int64_t N, int d, const float* C, int K,
                          const uint16_t* idx, float* R, hipStream_t st)
{
    const int64_t total = M * N;
    TimedRegion tr("residual", K, st);
    if (d == 8 && aligned16(X) && aligned16(C) && aligned16(R)) {
        const int64_t n_half = total / 4;
        hipLaunchKernelGGL(k_residual8, dim3(grid_for(n_half, kBlock)), dim3(kBlock), 0, st,
                           reinterpret_cast<const float4*>(X), n_half, reinterpret_cast<const float4*>(C), K,
                           idx, reinterpret_cast<float4*>(R));
        VQ_LAUNCHED("k_residual8");
        return VQ_OK;
    }
    hipLaunchKernelGGL(k_residual, dim3(grid_for(total, kBlock)), dim3(kBlock), 0, st, X, total, d, C, K,
                       idx, R);
    VQ_LAUNCHED("k_residual");
    return VQ_OK;
}

vq_status reconstruct_launch(int64_t M, int64_t N, int d, const float* C1, int K1, const uint16_t* idx1,
                             const float* C2, int K2, const uint16_t* idx2, const float* rs,
                             const float* cs, const int32_t* row_ptr, const int32_t* col,
                             const float* val, float* Wh, hipStream_t st)
{
    const int64_t n_sub = M * N / d;
    TimedRegion tr("reconstruct", K1, st);
    constexpr int kU = 4;                                        // halves per thread in k_decode8u
    const int64_t bpr = (2 * (N / d) + kBlock * kU - 1) / (kBlock * kU);   // workgroups per row
    if (d == 8 && aligned16(C1) && aligned16(C2) && aligned16(cs) && aligned16(Wh) && M * bpr <= (int64_t)UINT32_MAX) {
        const float4* c1 = reinterpret_cast<const float4*>(C1);
        const float4* c2 = reinterpret_cast<const float4*>(C2);
        const float4* c4 = reinterpret_cast<const float4*>(cs);
        float4* w4 = reinterpret_cast<float4*>(Wh);
        if (C2 && K2 <= kC2Lds) {
            hipLaunchKernelGGL((k_decode8u<kU, true>), dim3((unsigned)(M * bpr)), dim3(kBlock), 0, st, N / d,
                               (unsigned)bpr, c1, K1, idx1, c2, K2, idx2, rs, c4, w4);
        } else {
            hipLaunchKernelGGL((k_decode8u<kU, false>), dim3((unsigned)(M * bpr)), dim3(kBlock), 0, st, N / d,
                               (unsigned)bpr, c1, K1, idx1, c2, K2, idx2, rs, c4, w4);
        }
        VQ_LAUNCHED("k_decode8u");
    } else {
        hipLaunchKernelGGL(k_decode, dim3(grid_for(n_sub, kBlock)), dim3(kBlock), 0, st, n_sub, N / d, d,
                           C1, K1, idx1, C2, K2, idx2, rs, cs, Wh);
        VQ_LAUNCHED("k_decode");
    }
    if (row_ptr) {
        if (M > (int64_t)UINT32_MAX) return fail(VQ_ERR_UNSUPPORTED, "vq_reconstruct: too many rows");
        hipLaunchKernelGGL(k_sparse_overwrite, dim3((unsigned)M), dim3(kBlock), 0, st, N, row_ptr, col, val, Wh);
        VQ_LAUNCHED("k_sparse_overwrite");
    }
    return VQ_OK;
}

vq_status sparse_overwrite_launch(int64_t M, int64_t N, const int32_t* row_ptr, const int32_t* col,
                                  const float* val, float* Wh, hipStream_t st)
{
    if (M > (int64_t)UINT32_MAX) return fail(VQ_ERR_UNSUPPORTED, "sparse overwrite: too many rows");
    hipLaunchKernelGGL(k_sparse_overwrite, dim3((unsigned)M), dim3(kBlock), 0, st, N, row_ptr, col, val, Wh);
    VQ_LAUNCHED("k_sparse_overwrite");
    return VQ_OK;
}

vq_status objective_launch(const float* X, const float* hcol, const float* rho, const uint8_t* mask,
                           int64_t M, int64_t N, int d, const float* C, int K, const uint16_t* idx,
                           double* J, void* ws, size_t ws_bytes, hipStream_t st)
{
    const int64_t n_sub = M * N / d;
    const unsigned nblk = grid_for(n_sub, kObjPerBlock);
    Carver cv(ws, ws_bytes);
    double* part = cv.take<double>(nblk);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_objective: workspace too small");
    TimedRegion tr("objective", K, st);
    const int vec = (d == 8 && aligned16(X) && aligned16(C) && aligned16(hcol)) ? 1 : 0;
    hipLaunchKernelGGL(k_objective_partial, dim3(nblk), dim3(kBlock), 0, st, X, hcol, rho, mask, n_sub,
                       (uint32_t)(N / d), d, C, K, idx, vec, part);
    VQ_LAUNCHED("k_objective_partial");
    hipLaunchKernelGGL(k_sum_partials, dim3(1), dim3(1024), 0, st, part, (int64_t)nblk, J);
    VQ_LAUNCHED("k_sum_partials");
    return VQ_OK;
}

}  // namespace vq
