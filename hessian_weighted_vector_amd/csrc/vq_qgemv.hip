// Fused dequantize-and-multiply: Y = X * W_hat^T straight from the compressed
// form (indices, codebooks, row/column scales, sparse correction), never
// writing W_hat.  VPTQ page, "End-to-End Quantization Pipeline": at inference
// the weights are decoded by codebook lookup inside the matrix-vector product;
// SCVQ summary: the exact sparse term is applied in the same product.
//
// Work split.  The columns are cut into slabs of whole sub-vectors, sized so
// that the slab of scaled activations x'_bj = x_bj * cscale_j of every token
// in the launch fits in LDS (each workgroup stages it once and every row
// reuses it).  A workgroup owns one slab and a group of rows; each wave walks
// one row at a time.  For d = 8 a lane pair owns a sub-vector per step (each
// lane half of it): coalesced index loads, one gather instruction that
// fetches 32 whole centroid rows from C1 (L2-resident), the residual rows from
// LDS when the residual codebook is small, and 4 fused multiply-adds per lane
// and token.  The row's salient entries that fall in the slab
// are applied by the same wave afterwards: the decoded weight's term is taken
// back out and val * x added.  A fixed shuffle tree sums the wave; with more
// than one slab the partial sums go to the workspace and a second kernel adds
// them in slab order, so every result is bitwise reproducible.
#include "vq_internal.h"

namespace vq {
namespace {

constexpr int kQThreads = 512;                 // 8 waves per workgroup
constexpr int kQWaves = kQThreads / 64;
constexpr int kXsFloats = 14336;               // LDS for the scaled activations (56 KB)
constexpr int kC2LdsFloats = 2048;             // residual codebooks up to 8 KB are held in LDS
constexpr int kMaxTokens = 8;                  // tokens per launch

__device__ inline float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// D = 8: the centroid rows are read as two float4 (C1, C2, X and cscale
// 16-byte aligned).  D = 0: any d in [1, 8], scalar loads.
// C2M: 0 = no residual stage, 1 = residual codebook staged in LDS, 2 = read
// from global memory.
template <int D, int TB, int C2M>
__global__ __launch_bounds__(kQThreads) void k_qgemv(
    int64_t M, int64_t N, int d_rt, int64_t nb, int sb,
    const float* __restrict__ C1, const uint16_t* __restrict__ idx1,
    const float* __restrict__ C2, int K2, const uint16_t* __restrict__ idx2,
    const float* __restrict__ rs, const float* __restrict__ cs,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col, const float* __restrict__ val,
    const float* __restrict__ X, int rows_per_wg, float* __restrict__ out, int64_t slab_stride)
{
    extern __shared__ float lds[];
    const int d = D > 0 ? D : d_rt;
    const int sbd = sb * d;                      // LDS row length of one token
    float* xs = lds;                             // [TB][sbd]
    float* c2s = lds + TB * sbd;                 // [K2 * d] when C2M == 1

    const int slab = blockIdx.y;
    const int64_t s0 = (int64_t)slab * sb;
    const int nsv = (int)(nb - s0 < (int64_t)sb ? nb - s0 : (int64_t)sb);
    const int ncol = nsv * d;
    const int64_t c0 = s0 * d;

    // stage x' = x * cscale for the slab (and the residual codebook)
    if (D == 8) {
        const int nq = ncol / 4;
        for (int b = 0; b < TB; ++b) {
            const float4* xr = reinterpret_cast<const float4*>(X + b * N + c0);
            float4* xw = reinterpret_cast<float4*>(xs + b * sbd);
            for (int q = threadIdx.x; q < nq; q += kQThreads) {
                float4 v = xr[q];
                if (cs) {
                    const float4 c = reinterpret_cast<const float4*>(cs + c0)[q];
                    v.x = v.x * c.x; v.y = v.y * c.y; v.z = v.z * c.z; v.w = v.w * c.w;
                }
                xw[q] = v;
            }
        }
    } else {
        for (int b = 0; b < TB; ++b)
            for (int j = threadIdx.x; j < ncol; j += kQThreads) {
                const float v = X[b * N + c0 + j];
                xs[b * sbd + j] = cs ? v * cs[c0 + j] : v;
            }
    }
    if (C2M == 1)
        for (int k = threadIdx.x; k < K2 * d; k += kQThreads) c2s[k] = C2[k];
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_wg;
    const int64_t r1 = r0 + rows_per_wg < M ? r0 + rows_per_wg : M;
    for (int64_t i = r0 + wave; i < r1; i += kQWaves) {
        const uint16_t* ir1 = idx1 + i * nb + s0;
        const uint16_t* ir2 = idx2 + i * nb + s0;
        float acc[TB];
#pragma unroll
        for (int b = 0; b < TB; ++b) acc[b] = 0.0f;

        if (D == 8) {
            // lane pairs share a sub-vector: the even lane takes elements 0-3,
            // the odd lane 4-7, so one load instruction fetches whole centroid
            // rows (one cache-line request per sub-vector) and every lane keeps
            // a partial sum over its half
            const int h = lane & 1;
#pragma unroll 8
            for (int s = lane >> 1; s < nsv; s += 32) {
                float4 w = reinterpret_cast<const float4*>(C1)[2 * (int)ir1[s] + h];
                if (C2M != 0) {
                    const int k2 = ir2[s];
                    const float4 w2 = C2M == 1 ? reinterpret_cast<const float4*>(c2s)[2 * k2 + h]
                                               : reinterpret_cast<const float4*>(C2)[2 * k2 + h];
                    w.x = w.x + w2.x; w.y = w.y + w2.y; w.z = w.z + w2.z; w.w = w.w + w2.w;
                }
#pragma unroll
                for (int b = 0; b < TB; ++b) {
                    const float4 xv = reinterpret_cast<const float4*>(xs + b * sbd)[2 * s + h];
                    float a = acc[b];
                    a = fmaf(w.x, xv.x, a); a = fmaf(w.y, xv.y, a);
                    a = fmaf(w.z, xv.z, a); a = fmaf(w.w, xv.w, a);
                    acc[b] = a;
                }
            }
        } else {
            for (int s = lane; s < nsv; s += 64) {
                const float* c1 = C1 + (size_t)ir1[s] * d;
                const float* c2 = nullptr;
                if (C2M != 0) c2 = (C2M == 1 ? c2s : C2) + (size_t)ir2[s] * d;
                for (int t = 0; t < d; ++t) {
                    float w = c1[t];
                    if (C2M != 0) w = w + c2[t];
#pragma unroll
                    for (int b = 0; b < TB; ++b) acc[b] = fmaf(w, xs[b * sbd + s * d + t], acc[b]);
                }
            }
        }

        // salient entries of this row inside the slab: remove the decoded
        // weight's term, add the exact value's
        float sp[TB];
#pragma unroll
        for (int b = 0; b < TB; ++b) sp[b] = 0.0f;
        if (row_ptr) {
            const int e1 = row_ptr[i + 1];
            for (int e = row_ptr[i] + lane; e < e1; e += 64) {
                const int64_t jj = (int64_t)col[e] - c0;
                if (jj < 0 || jj >= ncol) continue;
                const int sv = (int)(jj / d);
                const int t = (int)(jj - (int64_t)sv * d);
                float w = C1[(size_t)ir1[sv] * d + t];
                if (C2M != 0) w = w + (C2M == 1 ? c2s : C2)[(size_t)ir2[sv] * d + t];
                const float v = val[e];
#pragma unroll
                for (int b = 0; b < TB; ++b) {
                    acc[b] = fmaf(-w, xs[b * sbd + jj], acc[b]);
                    sp[b] = fmaf(v, X[b * N + c0 + jj], sp[b]);
                }
            }
        }

        const float ri = rs ? rs[i] : 1.0f;
        float* o = out + slab * slab_stride;
#pragma unroll
        for (int b = 0; b < TB; ++b) {
            const float z = wave_sum(rs ? fmaf(ri, acc[b], sp[b]) : acc[b] + sp[b]);
            if (lane == 0) o[b * M + i] = z;
        }
    }
}

// Y[e] = sum over slabs of part[slab * stride + e], slabs in order.
__global__ __launch_bounds__(256) void k_qgemv_sum(const float* __restrict__ part, int nslab, int64_t stride,
                                                   int64_t n, float* __restrict__ Y)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= n) return;
    float s = part[e];
    for (int k = 1; k < nslab; ++k) s = s + part[k * stride + e];
    Y[e] = s;
}

struct QPlan {
    int tb, sb, nslab, rows_per_wg;
    unsigned groups;
};

QPlan qgemv_plan(int64_t M, int64_t N, int d, int tb)
{
    const int64_t nb = N / d;
    int64_t cap = kXsFloats / (tb * d);              // sub-vectors per slab that fit
    if (cap < 1) cap = 1;
    const int64_t nslab = (nb + cap - 1) / cap;
    const int64_t sb = (nb + nslab - 1) / nslab;     // balanced slabs
    QPlan p;
    p.tb = tb;
    p.sb = (int)sb;
    p.nslab = (int)nslab;
    p.rows_per_wg = kQWaves * tb;                    // activation staging amortized over more rows per token
    p.groups = (unsigned)((M + p.rows_per_wg - 1) / p.rows_per_wg);
    return p;
}

int chunk_tokens(int64_t left) { return left >= 8 ? 8 : left >= 4 ? 4 : left >= 2 ? 2 : 1; }

template <int D, int TB>
vq_status launch_tb(const QPlan& p, int c2m, int64_t M, int64_t N, int d, const float* C1,
                    const uint16_t* idx1, const float* C2, int K2, const uint16_t* idx2, const float* rs,
                    const float* cs, const int32_t* row_ptr, const int32_t* col, const float* val,
                    const float* X, float* out, int64_t slab_stride, hipStream_t st)
{
    const size_t lds = (size_t)(TB * p.sb * d + (c2m == 1 ? K2 * d : 0)) * sizeof(float);
    const dim3 grid(p.groups, (unsigned)p.nslab);
    const int64_t nb = N / d;
#define VQ_QG_LAUNCH(C2M_)                                                                                  \
    hipLaunchKernelGGL((k_qgemv<D, TB, C2M_>), grid, dim3(kQThreads), lds, st, M, N, d, nb, p.sb, C1, idx1, \
                       C2, K2, idx2, rs, cs, row_ptr, col, val, X, p.rows_per_wg, out, slab_stride)
    if (c2m == 0) VQ_QG_LAUNCH(0);
    else if (c2m == 1) VQ_QG_LAUNCH(1);
    else VQ_QG_LAUNCH(2);
#undef VQ_QG_LAUNCH
    VQ_LAUNCHED("k_qgemv");
    return VQ_OK;
}

template <int D>
vq_status launch_d(const QPlan& p, int c2m, int64_t M, int64_t N, int d, const float* C1,
                   const uint16_t* idx1, const float* C2, int K2, const uint16_t* idx2, const float* rs,
                   const float* cs, const int32_t* row_ptr, const int32_t* col, const float* val,
                   const float* X, float* out, int64_t slab_stride, hipStream_t st)
{
    switch (p.tb) {
    case 1: return launch_tb<D, 1>(p, c2m, M, N, d, C1, idx1, C2, K2, idx2, rs, cs, row_ptr, col, val, X, out, slab_stride, st);
    case 2: return launch_tb<D, 2>(p, c2m, M, N, d, C1, idx1, C2, K2, idx2, rs, cs, row_ptr, col, val, X, out, slab_stride, st);
    case 4: return launch_tb<D, 4>(p, c2m, M, N, d, C1, idx1, C2, K2, idx2, rs, cs, row_ptr, col, val, X, out, slab_stride, st);
    default: return launch_tb<D, 8>(p, c2m, M, N, d, C1, idx1, C2, K2, idx2, rs, cs, row_ptr, col, val, X, out, slab_stride, st);
    }
}

}  // namespace

size_t ws_qgemv(int64_t M, int64_t N, int d, int64_t B)
{
    size_t need = 0;
    for (int tb = 1; tb <= kMaxTokens; tb *= 2) {
        if (tb > B && tb > 1) break;
        const QPlan p = qgemv_plan(M, N, d, tb);
        if (p.nslab > 1) {
            const size_t b = align_up((size_t)p.nslab * (size_t)tb * (size_t)M * sizeof(float));
            if (b > need) need = b;
        }
    }
    return need;
}

vq_status qgemv_launch(int64_t M, int64_t N, int d, const float* C1, int K1, const uint16_t* idx1,
                       const float* C2, int K2, const uint16_t* idx2, const float* rs, const float* cs,
                       const int32_t* row_ptr, const int32_t* col, const float* val, const float* X,
                       int64_t B, float* Y, void* ws, size_t ws_bytes, hipStream_t st)
{
    if (B == 0) return VQ_OK;
    const bool vec = d == 8 && aligned16(C1) && aligned16(X) && (!cs || aligned16(cs)) &&
                     (!C2 || aligned16(C2));
    const int c2m = C2 == nullptr ? 0 : ((int64_t)K2 * d <= kC2LdsFloats ? 1 : 2);
    TimedRegion tr("qgemv", K1, st);
    for (int64_t b0 = 0; b0 < B;) {
        const int tb = chunk_tokens(B - b0);
        const QPlan p = qgemv_plan(M, N, d, tb);
        if (p.groups == 0 || (int64_t)p.groups * p.rows_per_wg < M)
            return fail(VQ_ERR_UNSUPPORTED, "vq_qgemv: too many rows");
        float* out = Y + b0 * M;
        float* part = nullptr;
        const int64_t stride = (int64_t)tb * M;
        if (p.nslab > 1) {
            Carver cv(ws, ws_bytes);
            part = cv.take<float>((size_t)p.nslab * (size_t)stride);
            if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_qgemv: workspace too small");
        }
        const float* Xc = X + b0 * N;
        float* dst = part ? part : out;
        vq_status r = vec ? launch_d<8>(p, c2m, M, N, d, C1, idx1, C2, K2, idx2, rs, cs, row_ptr, col, val, Xc,
                                        dst, stride, st)
                          : launch_d<0>(p, c2m, M, N, d, C1, idx1, C2, K2, idx2, rs, cs, row_ptr, col, val, Xc,
                                        dst, stride, st);
        if (r != VQ_OK) return r;
        if (part) {
            hipLaunchKernelGGL(k_qgemv_sum, dim3(grid_for(stride, 256)), dim3(256), 0, st, part, p.nslab, stride,
                               stride, out);
            VQ_LAUNCHED("k_qgemv_sum");
        }
        b0 += tb;
    }
    return VQ_OK;
}

}  // namespace vq
