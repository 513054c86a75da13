// Weighted nearest-centroid assignment for gfx950.
//
// Method: VPTQ page, "The Core Algorithm" (Q_V: nearest centroid per vector)
// under the diagonal-Hessian weighting of "Hessian-Weighted Centroid
// Initialization": D(s,k) = sum_t omega_t (x_t - c_kt)^2.
//
// Design.  The row weight rho_i scales every D(s,.) of a sub-vector by the
// same positive factor, so the search ranks e(s,k) = D(s,k)/rho_i - S_s with
// S_s = sum_t omega_t x_t^2 (omega without rho), written as one inner product
// of length 2d = 16:
//     e(s,k) = < [omega (.) x, omega], [-2 c_k, c_k (.) c_k] >
// That is a skinny GEMM (sub-vectors x 16) . (16 x centroids), run on the
// fp32 matrix cores: v_mfma_f32_32x32x2f32, A = 32 centroids, B = 32
// sub-vectors, 8 instructions per 32x32 tile of pairs.  Each lane of the
// 32x32 accumulator holds 16 centroid rows of one sub-vector, so the running
// argmin needs no cross-lane traffic: per accumulator slot it keeps the best
// value, the second-best value and the tile of the best (4 VALU ops per
// pair: compare, min, select, median-of-three).
//
// Exactness.  Eight chained 32x32x2 fp32 MFMAs round like a sequential
// fused-multiply-add chain over the 16 terms, so |e~ - e| <= 17u sum|terms|
// (u = 2^-24, one more u for rounding omega*x and c*c).  Using
// sum|terms| <= 9 S + 4 e, a winner is certified when the gap to the second
// best exceeds the sum of both bounds (taken with a factor ~2 margin).
// Certified winners are the exact argmin; the rest are re-searched in
// float64 with the direct form in t order (k_assign_exact), which rounds
// exactly like a plain float64 implementation, ties to the lowest index.
#include "vq_internal.h"

#include <algorithm>

namespace vq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kSubPerWave = 32;           // sub-vectors per wave (MFMA B columns)
constexpr int kSubPerBlock = kWaves * kSubPerWave;
constexpr int kTile = 32;                 // centroids per MFMA tile (A rows)
constexpr int kChunkTiles = 8;            // tiles staged in LDS at once
constexpr float kPadSq = 1.0e30f;         // c*c of padding centroids
constexpr int kExactBlocks = 2048;

// P[k] = 16 floats: [-2 c_k0..-2 c_k7, c_k0^2..c_k7^2]; dims >= d are 0;
// padding centroids (k >= K) have -2c = 0 and c^2 = kPadSq.  Also clears
// the flag counter for the following search.
__global__ void k_cb_prep(const float* __restrict__ C, int K, int d, int Kpad,
                          float* __restrict__ P, int* __restrict__ flag_count)
{
    int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k == 0) *flag_count = 0;
    if (k >= Kpad) return;
    float* p = P + (size_t)k * 16;
    for (int t = 0; t < 8; ++t) {
        float m2c = 0.f, sq = 0.f;
        if (k < K) {
            if (t < d) {
                float c = C[(size_t)k * d + t];
                m2c = -2.f * c;
                sq = c * c;
            }
        } else {
            sq = kPadSq;
        }
        p[t] = m2c;
        p[8 + t] = sq;
    }
}

// The float64 direct form, in t order: acc += omega_t * ((x_t - c_t)^2).
__device__ inline double exact_dist(const double* om, const float* x, const float* c, int d)
{
    double acc = 0.0;
    for (int t = 0; t < d; ++t) {
        double diff = (double)x[t] - (double)c[t];
        double sq = diff * diff;
        acc = acc + om[t] * sq;
    }
    return acc;
}

// Weight of element t of sub-vector s in float64, exactly as a plain float64
// evaluation forms it: hcol (times rho if present), 0 when masked.
__device__ inline void exact_weights(const float* hcol, const float* rho, const uint8_t* mask,
                                     int64_t s, int64_t nb, int d, double* om)
{
    int64_t i = s / nb;
    int64_t b = s - i * nb;
    unsigned mb = mask ? mask[s] : 0u;
    for (int t = 0; t < d; ++t) {
        double w = (double)hcol[b * d + t];
        if (rho) w = w * (double)rho[i];
        om[t] = ((mb >> t) & 1u) ? 0.0 : w;
    }
}

__global__ __launch_bounds__(256) void k_assign_mfma(
    const float* __restrict__ X, const float* __restrict__ hcol, const float* __restrict__ rho,
    const uint8_t* __restrict__ mask, int64_t n_sub, int64_t nb, int d,
    const float4* __restrict__ P, const float* __restrict__ C, int K, int Kt,
    uint16_t* __restrict__ idx, float* __restrict__ dist,
    int* __restrict__ flag_count, int* __restrict__ flag_list)
{
    __shared__ float4 lds[kChunkTiles * kTile * 4];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int64_t s = (int64_t)blockIdx.x * kSubPerBlock + wave * kSubPerWave + (lane & 31);
    const bool valid = s < n_sub;

    // ---- the sub-vector's B operand and its weighted energy S ----------
    float x[8], om[8];
    float S = 0.f;
    {
        unsigned mb = (valid && mask) ? mask[s] : 0u;
        int64_t b = valid ? (s % nb) : 0;
        for (int t = 0; t < 8; ++t) {
            float xv = 0.f, w = 0.f;
            if (valid && t < d) {
                xv = X[s * d + t];
                w = ((mb >> t) & 1u) ? 0.f : hcol[b * d + t];
            }
            x[t] = xv;
            om[t] = w;
            S += w * xv * xv;
        }
    }
    float bv[8];
    for (int t = 0; t < 8; ++t) bv[t] = half ? om[t] : om[t] * x[t];

    float m1[16], m2[16];
    int i1[16];
    for (int j = 0; j < 16; ++j) {
        m1[j] = __builtin_inff();
        m2[j] = __builtin_inff();
        i1[j] = 0;
    }

    for (int c0 = 0; c0 < Kt; c0 += kChunkTiles) {
        const int nt = min(kChunkTiles, Kt - c0);
        __syncthreads();
        const float4* src = P + (size_t)c0 * kTile * 4;
        for (int q = threadIdx.x; q < nt * kTile * 4; q += blockDim.x) lds[q] = src[q];
        __syncthreads();
        for (int tt = 0; tt < nt; ++tt) {
            const float4* a4 = &lds[(tt * kTile + (lane & 31)) * 4 + half * 2];
            const float4 a0 = a4[0];
            const float4 a1 = a4[1];
            f32x16 acc = {};
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.x, bv[0], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.y, bv[1], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.z, bv[2], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.w, bv[3], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a1.x, bv[4], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a1.y, bv[5], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a1.z, bv[6], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a1.w, bv[7], acc, 0, 0, 0);
            const int kt = c0 + tt;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float v = acc[j];
                m2[j] = __builtin_amdgcn_fmed3f(m1[j], m2[j], v);
                const bool lt = v < m1[j];
                m1[j] = lt ? v : m1[j];
                i1[j] = lt ? kt : i1[j];
            }
        }
    }

    // ---- epilogue: best and second best of this sub-vector -------------
    // accumulator slot j of this lane holds centroid row (j/4)*8 + half*4 + j%4
    float b1 = m1[0];
    int bj = 0;
    for (int j = 1; j < 16; ++j)
        if (m1[j] < b1) { b1 = m1[j]; bj = j; }
    float sec = __builtin_inff();
    for (int j = 0; j < 16; ++j) sec = fminf(sec, j == bj ? m2[j] : m1[j]);
    int kb = 0;
    for (int j = 0; j < 16; ++j)
        if (j == bj) kb = i1[j] * kTile + (j >> 2) * 8 + half * 4 + (j & 3);

    const float ob1 = __shfl_xor(b1, 32);
    const float osec = __shfl_xor(sec, 32);
    const int okb = __shfl_xor(kb, 32);
    float gb, gs;
    int gk;
    if (b1 < ob1 || (b1 == ob1 && kb < okb)) {
        gb = b1; gk = kb; gs = fminf(sec, ob1);
    } else {
        gb = ob1; gk = okb; gs = fminf(osec, b1);
    }
    const float u = 5.9604644775390625e-8f;   // 2^-24
    const float eb = 32.f * u * (9.f * S + 4.f * fmaxf(gb, -S));
    const float es = 32.f * u * (9.f * S + 4.f * fmaxf(gs, -S));
    const bool certified = (gs - gb) > (eb + es + 1.0e-35f) && gk < K;

    const bool writer = valid && half == 0;
    if (writer && certified) {
        idx[s] = (uint16_t)gk;
        if (dist) {
            double omd[8];
            float xs[8];
            exact_weights(hcol, rho, mask, s, nb, d, omd);
            for (int t = 0; t < d; ++t) xs[t] = x[t];
            dist[s] = (float)exact_dist(omd, xs, C + (size_t)gk * d, d);
        }
    }
    // uncertified winners go to the exact search (one atomic per wave)
    const bool flag = writer && !certified;
    const unsigned long long ball = __ballot(flag);
    if (ball) {
        int base = 0;
        const int leader = __ffsll((long long)ball) - 1;
        if (lane == leader) base = atomicAdd(flag_count, __popcll(ball));
        base = __shfl(base, leader);
        if (flag) {
            const int rank = __popcll(ball & ((1ull << lane) - 1ull));
            flag_list[base + rank] = (int)s;
        }
    }
}

// Exact float64 re-search of the flagged sub-vectors: one workgroup per
// flagged sub-vector (grid-stride), lexicographic (D, k) minimum.
__global__ __launch_bounds__(256) void k_assign_exact(
    const float* __restrict__ X, const float* __restrict__ hcol, const float* __restrict__ rho,
    const uint8_t* __restrict__ mask, int64_t nb, int d, const float* __restrict__ C, int K,
    const int* __restrict__ flag_count, const int* __restrict__ flag_list,
    uint16_t* __restrict__ idx, float* __restrict__ dist)
{
    __shared__ double sd[256];
    __shared__ int sk[256];
    const int n = *flag_count;
    for (int f = blockIdx.x; f < n; f += gridDim.x) {
        const int64_t s = flag_list[f];
        double om[8];
        float x[8];
        exact_weights(hcol, rho, mask, s, nb, d, om);
        for (int t = 0; t < d; ++t) x[t] = X[s * d + t];
        double best = __builtin_inf();
        int arg = K;
        for (int k = threadIdx.x; k < K; k += blockDim.x) {
            const double v = exact_dist(om, x, C + (size_t)k * d, d);
            if (v < best) { best = v; arg = k; }
        }
        sd[threadIdx.x] = best;
        sk[threadIdx.x] = arg;
        __syncthreads();
        for (int w = blockDim.x / 2; w > 0; w >>= 1) {
            if ((int)threadIdx.x < w) {
                const double ov = sd[threadIdx.x + w];
                const int ok = sk[threadIdx.x + w];
                if (ov < sd[threadIdx.x] || (ov == sd[threadIdx.x] && ok < sk[threadIdx.x])) {
                    sd[threadIdx.x] = ov;
                    sk[threadIdx.x] = ok;
                }
            }
            __syncthreads();
        }
        if (threadIdx.x == 0) {
            idx[s] = (uint16_t)sk[0];
            if (dist) dist[s] = (float)sd[0];
        }
        __syncthreads();
    }
}

}  // namespace

size_t ws_assign(int64_t n_sub, int K)
{
    const int64_t Kt = (K + kTile - 1) / kTile;
    return align_up((size_t)Kt * kTile * 16 * sizeof(float)) + align_up(sizeof(int)) +
           align_up((size_t)n_sub * sizeof(int));
}

// Enqueues the assignment; arguments already validated by the caller.
vq_status assign_launch(const float* X, const float* hcol, const float* rho, const uint8_t* mask,
                        int64_t M, int64_t N, int d, const float* C, int K,
                        uint16_t* idx, float* dist, void* ws, size_t ws_bytes, hipStream_t st)
{
    const int64_t n_sub = M * N / d;
    const int64_t nb = N / d;
    const int Kt = (K + kTile - 1) / kTile;
    Carver cv(ws, ws_bytes);
    float* P = cv.take<float>((size_t)Kt * kTile * 16);
    int* flag_count = cv.take<int>(1);
    int* flag_list = cv.take<int>((size_t)n_sub);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_assign: workspace too small");

    const int Kpad = Kt * kTile;
    TimedRegion tr_all("assign", K, st);
    hipLaunchKernelGGL(k_cb_prep, dim3(grid_for(Kpad, 256)), dim3(256), 0, st, C, K, d, Kpad, P,
                       flag_count);
    VQ_LAUNCHED("k_cb_prep");
    {
        TimedRegion tr("assign_search", K, st);
        hipLaunchKernelGGL(k_assign_mfma, dim3(grid_for(n_sub, kSubPerBlock)), dim3(256), 0, st, X, hcol,
                           rho, mask, n_sub, nb, d, reinterpret_cast<const float4*>(P), C, K, Kt, idx, dist,
                           flag_count, flag_list);
        VQ_LAUNCHED("k_assign_mfma");
    }
    const unsigned gx = (unsigned)std::min<int64_t>(n_sub, kExactBlocks);
    hipLaunchKernelGGL(k_assign_exact, dim3(gx), dim3(256), 0, st, X, hcol, rho, mask, nb, d, C, K,
                       flag_count, flag_list, idx, dist);
    VQ_LAUNCHED("k_assign_exact");
    return VQ_OK;
}

// Number of sub-vectors the last search sent to the exact path (diagnostics).
vq_status assign_flag_count(void* ws, size_t ws_bytes, int64_t n_sub, int K, int* out, hipStream_t st)
{
    const int Kt = (K + kTile - 1) / kTile;
    Carver cv(ws, ws_bytes);
    cv.take<float>((size_t)Kt * kTile * 16);
    int* flag_count = cv.take<int>(1);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "workspace too small");
    VQ_HIP(hipMemcpyAsync(out, flag_count, sizeof(int), hipMemcpyDeviceToHost, st));
    VQ_HIP(hipStreamSynchronize(st));
    (void)n_sub;
    return VQ_OK;
}

}  // namespace vq
