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
//     e(s,k) = < [omega (.) x, omega], [-2 c_k, c_k (.) c_k] >.
// That is a skinny GEMM (centroids x 16) . (16 x sub-vectors).  It runs on
// the fp16 matrix cores (v_mfma_f32_32x32x16_f16, fp32 accumulation) with
// every fp32 operand split into two fp16 parts after an exact power-of-two
// scaling: the codebook side by one factor per term kind for the whole
// codebook, the sub-vector side by one factor per sub-vector, so each side's
// largest value lies in [2^14, 2^15) (no overflow; small parts may be fp16
// subnormals, which the conversion forms and the matrix cores multiply
// exactly).  A tile of 32 centroids x 32 sub-vectors takes three MFMAs,
// lo*hi and hi*lo first and hi*hi last:
//     e~ = sum_t (al bh + ah bl + ah bh)   (the lo*lo product is dropped).
// The per-sub-vector factor does not change the ranking.  Each lane of the
// accumulator holds 16 centroid rows of one sub-vector, so the running
// argmin needs no cross-lane traffic: per lane it keeps the best value,
// the second-best value and the position of the best.
//
// Exactness.  With u = 2^-24: splitting leaves |a - ah - al| <= 2^-22 |a|
// (two 11-bit parts), so the three products miss at most 12.1u|ab| of each
// term; the fp32 terms omega*x and c*c carry one rounding (u); the first two
// MFMAs sum products that are 2^-11 smaller, and the last one adds 16
// products with fp32 roundings, at most 16u (round to nearest) or 32u
// (truncation) of sum|terms| whatever the order of its additions: 45.2u in
// all.  Rounding in fp16's subnormal range adds at most 2^-25 per part,
// under 2^-5 per pair in scaled units.  Using sum|terms| <= 9 S + 4 e, a
// winner is certified when the gap to the second best exceeds
// 48u (9 S + 4 e) + 1 for both of them.  Certified winners are the exact
// argmin; the rest are re-searched in float64 with the direct form in t
// order (k_assign_exact), which rounds exactly like a plain float64
// implementation, ties to the lowest index.
#include "vq_internal.h"

#include <algorithm>

namespace vq {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 8;                 // waves per workgroup
constexpr int kSubPerWave = 32;           // sub-vectors per wave (MFMA B columns)
constexpr int kSubPerBlock = kWaves * kSubPerWave;
constexpr int kTile = 32;                 // centroids per MFMA tile (A rows)
constexpr int kChunkTiles = 8;            // tiles staged in LDS at once
constexpr int kExactBlocks = 2048;
constexpr int kSlotChunks = 8;            // codebooks of <= 8 chunks use per-slot tracking
constexpr float kPadSq = 16384.0f;           // scaled c*c term of padding centroids

constexpr int kMaxBlocks = 256;   // blocks of the codebook max reduction

// Largest |C| over the codebook, two passes: block maxima into part[], then
// one block reduces them into *cmax and clears the flag and dirty counters.
__global__ __launch_bounds__(256) void k_cb_absmax_part(const float* __restrict__ C, int64_t n,
                                                        float* __restrict__ part)
{
    __shared__ float red[256];
    float m = 0.f;
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < n; q += (int64_t)gridDim.x * 256)
        m = fmaxf(m, fabsf(C[q]));
    red[threadIdx.x] = m;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
        __syncthreads();
    }
    if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void k_cb_absmax_final(const float* __restrict__ part, int nparts,
                                                         float* __restrict__ cmax, int* __restrict__ flag_count,
                                                         int* __restrict__ dirty_count)
{
    __shared__ float red[256];
    red[threadIdx.x] = (int)threadIdx.x < nparts ? part[threadIdx.x] : 0.f;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        *cmax = red[0];
        *flag_count = 0;
        *dirty_count = 0;
    }
}

// Binary exponents of the codebook scale factors from the largest |c|:
// beta = 2^(15 - e1) puts max|2c| in [2^14, 2^15), beta2 = 2^(15 - e2) does
// the same for max c*c.
__device__ inline void cb_exponents(float cmax, int& e1, int& e2)
{
    frexpf(2.f * cmax, &e1);
    frexpf(cmax * cmax, &e2);
}

// Splits a scaled fp32 value into fp16 parts hi + lo, both rounded to
// nearest (fp16 subnormals included: the conversion produces them and the
// matrix cores multiply them exactly).
__device__ inline void split_h16(float v, _Float16& hi, _Float16& lo)
{
    const _Float16 h = (_Float16)v;
    hi = h;
    lo = (_Float16)(v - (float)h);
}

// Expanded, scaled and split codebook.  Per tile of 32 centroids, 4 rows of
// 32 x 16 bytes: (hi, terms 0-7), (hi, terms 8-15), (lo, terms 0-7),
// (lo, terms 8-15), where term t < 8 is -2 beta c_t and term 8 + t is
// beta2 c_t^2.  Centroid m of the tile sits at position m of each row, so
// the 64 lanes of a wavefront read one row pair as 1 KB of consecutive
// bytes.  Dimensions >= d are 0; padding centroids (k >= K) have 0 cross
// terms and kPadSq square terms.
__global__ void k_cb_prep16(const float* __restrict__ C, int K, int d, int Kpad, const float* __restrict__ cmax,
                            uint4* __restrict__ P)
{
    const int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= Kpad) return;
    int e1, e2;
    cb_exponents(*cmax, e1, e2);
    _Float16 hv[2][16];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        float m2c = 0.f, sq = 0.f;
        if (k < K) {
            if (t < d) {
                const float c = C[(size_t)k * d + t];
                m2c = ldexpf(-2.f * c, 15 - e1);
                sq = ldexpf(c * c, 15 - e2);
            }
        } else {
            sq = kPadSq;
        }
        split_h16(m2c, hv[0][t], hv[1][t]);
        split_h16(sq, hv[0][8 + t], hv[1][8 + t]);
    }
    const int tile = k / kTile, m = k % kTile;
#pragma unroll
    for (int part = 0; part < 2; ++part)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            h16x8 v;
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = hv[part][half * 8 + i];
            P[(size_t)tile * 128 + (part * 2 + half) * 32 + m] = __builtin_bit_cast(uint4, v);
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

// Minimum of a tile's 16 accumulator values: five three-way minima of the
// raw values, then two of their results, then one pair (seven v_min3 and one
// v_min; no operand of a two-way minimum is a raw accumulator value).
__device__ __forceinline__ float tile_min(const f32x16& a)
{
    const float m0 = fminf(fminf(a[0], a[1]), a[2]);
    const float m1 = fminf(fminf(a[3], a[4]), a[5]);
    const float m2 = fminf(fminf(a[6], a[7]), a[8]);
    const float m3 = fminf(fminf(a[9], a[10]), a[11]);
    const float m4 = fminf(fminf(a[12], a[13]), a[14]);
    const float n0 = fminf(fminf(m0, m1), m2);
    const float n1 = fminf(fminf(m3, m4), a[15]);
    return fminf(n0, n1);
}

// Per-lane tracking over tiles, branch-free: b1 = smallest tile minimum so
// far and kt1 its tile (the earlier tile on equal minima), b2 = smallest
// minimum of every other tile.  b1 <= b2 always, so b2' = med3(b1, tm, b2).
__device__ __forceinline__ void tile_track(const f32x16& a, int kt, float& b1, float& b2, int& kt1)
{
    const float tm = tile_min(a);
    b2 = __builtin_amdgcn_fmed3f(b1, tm, b2);
    const bool lt = tm < b1;
    b1 = lt ? tm : b1;
    kt1 = lt ? kt : kt1;
}

// x and its weights omega (hcol, zero where masked) of sub-vector s; zeros
// for an invalid lane and for dimensions >= d.  16-byte loads when d == 8
// and the buffers allow; n_sub < 2^31, so 32-bit index arithmetic.
__device__ __forceinline__ void load_sub(const float* __restrict__ X, const float* __restrict__ hcol,
                                         const uint8_t* __restrict__ mask, int64_t s, int64_t nb, int d, bool valid,
                                         bool vec, float (&x)[8], float (&w)[8])
{
#pragma unroll
    for (int t = 0; t < 8; ++t) { x[t] = 0.f; w[t] = 0.f; }
    if (!valid) return;
    const uint32_t su = (uint32_t)s;
    const uint32_t b = su % (uint32_t)nb;
    const unsigned mb = mask ? mask[s] : 0u;
    if (vec) {
        const float4 x0 = reinterpret_cast<const float4*>(X)[(size_t)su * 2];
        const float4 x1 = reinterpret_cast<const float4*>(X)[(size_t)su * 2 + 1];
        const float4 h0 = reinterpret_cast<const float4*>(hcol)[(size_t)b * 2];
        const float4 h1 = reinterpret_cast<const float4*>(hcol)[(size_t)b * 2 + 1];
        x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
        x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
        w[0] = h0.x; w[1] = h0.y; w[2] = h0.z; w[3] = h0.w;
        w[4] = h1.x; w[5] = h1.y; w[6] = h1.z; w[7] = h1.w;
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (t < d) {
                x[t] = X[(size_t)su * d + t];
                w[t] = hcol[(size_t)b * d + t];
            }
        }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t)
        if ((mb >> t) & 1u) w[t] = 0.f;
}

// Per-slot tracking (short codebooks, where a few branchy updates cost less
// than forming a tile again at the end): exact (best, second best, position
// = kt*16 + slot) over the 16 values of tile kt, in slot order (slot order is
// centroid order within the lane, so equal values keep the lower index).
// Only tiles whose minimum beats the second best are walked.
__device__ __forceinline__ void slot_track(const f32x16& a, int kt, float& b1, float& b2, int& kbp)
{
    if (tile_min(a) < b2) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float v = a[j];
            const bool lt = v < b1;
            b2 = __builtin_amdgcn_fmed3f(b1, b2, v);
            b1 = lt ? v : b1;
            kbp = lt ? kt * 16 + j : kbp;
        }
    }
}

template <bool SLOT>
__device__ __forceinline__ void track(const f32x16& a, int kt, float& b1, float& b2, int& pos)
{
    if (SLOT)
        slot_track(a, kt, b1, b2, pos);
    else
        tile_track(a, kt, b1, b2, pos);
}

// One 32x32 tile: three chained MFMAs (lo*hi, hi*lo, then hi*hi), with the
// previous tile's tracking update between them.
template <bool SLOT>
__device__ __forceinline__ f32x16 tile_h16(const h16x8 ah, const h16x8 al, const h16x8 bh, const h16x8 bl,
                                           const f32x16& prev, int ktp, float& b1, float& b2, int& pos)
{
    f32x16 acc = {};
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, acc, 0, 0, 0);
    track<SLOT>(prev, ktp, b1, b2, pos);
#pragma unroll
    for (int g = 0; g < 3; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // four VALU
    }
    return acc;
}

// The majority mask byte of each column block (lowest byte on ties): the
// weight pattern shared by most of its sub-vectors.
__global__ __launch_bounds__(256) void k_block_pattern(const uint8_t* __restrict__ mask, int64_t M, int64_t nb,
                                                       uint8_t* __restrict__ pattern)
{
    __shared__ int cnt[256];
    __shared__ int best_c[256], best_p[256];
    cnt[threadIdx.x] = 0;
    __syncthreads();
    const int64_t b = blockIdx.x;
    for (int64_t i = threadIdx.x; i < M; i += 256) atomicAdd(&cnt[mask[i * nb + b]], 1);
    __syncthreads();
    best_c[threadIdx.x] = cnt[threadIdx.x];
    best_p[threadIdx.x] = threadIdx.x;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) {
            const int oc = best_c[threadIdx.x + w], op = best_p[threadIdx.x + w];
            if (oc > best_c[threadIdx.x] || (oc == best_c[threadIdx.x] && op < best_p[threadIdx.x])) {
                best_c[threadIdx.x] = oc;
                best_p[threadIdx.x] = op;
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) pattern[b] = (uint8_t)best_p[0];
}

// Sub-vectors whose mask byte differs from their block's pattern are listed
// for the general kernel: wavefront ballots, a workgroup prefix in LDS and
// one integer atomic per workgroup (the order of the list does not affect
// any result).
__global__ __launch_bounds__(1024) void k_dirty(const uint8_t* __restrict__ mask, const uint8_t* __restrict__ pattern,
                                                int64_t n_sub, uint32_t nb, int* __restrict__ count,
                                                int* __restrict__ list)
{
    constexpr int kItems = 4;
    __shared__ int wsum[kItems][16];
    __shared__ int base;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    bool take[kItems];
    unsigned long long ball[kItems];
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
        const int64_t s = ((int64_t)blockIdx.x * kItems + r) * 1024 + threadIdx.x;
        take[r] = false;
        if (s < n_sub) take[r] = mask[s] != pattern[(uint32_t)(s % nb)];
        ball[r] = __ballot(take[r]);
        if (lane == 0) wsum[r][wave] = __popcll(ball[r]);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int tot = 0;
        for (int r = 0; r < kItems; ++r)
            for (int w = 0; w < 16; ++w) tot += wsum[r][w];
        base = tot ? atomicAdd(count, tot) : 0;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
        if (take[r]) {
            int off = base + __popcll(ball[r] & ((1ull << lane) - 1ull));
            for (int q = 0; q < r; ++q)
                for (int w = 0; w < 16; ++w) off += wsum[q][w];
            for (int w = 0; w < wave; ++w) off += wsum[r][w];
            const int64_t s = ((int64_t)blockIdx.x * kItems + r) * 1024 + threadIdx.x;
            list[off] = (int)s;
        }
    }
}

// One 32x32 tile of the shared-weight form: two chained MFMAs (the small
// cross products, then hi*hi with the bias), with the previous tile's
// tracking update between them.
template <bool SLOT>
__device__ __forceinline__ f32x16 tile2_h16(const h16x8 a0, const h16x8 a1, const h16x8 b0, const h16x8 b1v,
                                            const f32x16& prev, int ktp, float& b1, float& b2, int& pos)
{
    f32x16 acc = {};
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1v, acc, 0, 0, 0);
    track<SLOT>(prev, ktp, b1, b2, pos);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // six VALU
    }
    return acc;
}

// Final merge and certification of one lane pair (the two halves of a
// wavefront column), shared by both search kernels.  b1, b2 and pos come from
// the tracking; S_sc and shift_s are the sub-vector's scaled energy and
// scale; a writer lane that is not certified (or is marked bad) is appended
// to the exact re-search list.  A sub-vector whose weights are all zero has
// D = 0 for every centroid: index 0 (allzero, or found from its weights).
template <bool SLOT>
__device__ __forceinline__ void search_epilogue(
    const float* __restrict__ X, const float* __restrict__ hcol, const float* __restrict__ rho,
    const uint8_t* __restrict__ mask, int64_t nb, int d, const float* __restrict__ C, int K, int64_t s,
    bool valid, bool writer_ok, bool bad, bool allzero, int lane, int half, float b1, float b2, int kt1, float S_sc,
    int shift_s, uint16_t* __restrict__ idx, float* __restrict__ dist, int* __restrict__ flag_count,
    int* __restrict__ flag_list)
{
    // ---- epilogue: best and second best of this sub-vector -------------
    // Slot j of this lane holds centroid row (j/4)*8 + half*4 + j%4 of a tile,
    // rows ascending with j.  Per-slot tracking knows the best position
    // (kt1 = tile*16 + slot).  Per-tile tracking knows the best tile: its 16
    // values of this lane are formed again in fp32 (a fused multiply-add chain
    // over the 16 terms: within 17u of exact, inside the search's bound) to
    // find the best slot (the first minimum: lowest index) and the tile's
    // second best.
    float v1 = __builtin_inff(), v2 = __builtin_inff();
    int kb = K;
    const bool vecX = d == 8 && ((reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(hcol)) & 15u) == 0;
    {
        float xz[8], wz[8];
        load_sub(X, hcol, mask, s, nb, d, valid, vecX, xz, wz);
        bool z = true;
#pragma unroll
        for (int t = 0; t < 8; ++t) z = z && wz[t] == 0.f;
        allzero = allzero || z;
    }
    if (SLOT) {
        const int jb = kt1 & 15;
        kb = (kt1 >> 4) * kTile + (jb >> 2) * 8 + half * 4 + (jb & 3);
        v1 = b1;
    } else {
        float bw[8], om[8], xs[8];
        load_sub(X, hcol, mask, s, nb, d, valid, vecX, xs, om);
#pragma unroll
        for (int t = 0; t < 8; ++t) bw[t] = om[t] * xs[t];
        const bool vecC = d == 8 && (reinterpret_cast<uintptr_t>(C) & 15u) == 0;
#pragma unroll 2
        for (int j = 0; j < 16; ++j) {
            const int k = kt1 * kTile + (j >> 2) * 8 + half * 4 + (j & 3);
            if (k >= K) continue;
            float c[8];
            if (vecC) {
                const float4 ca = reinterpret_cast<const float4*>(C)[(size_t)k * 2];
                const float4 cb = reinterpret_cast<const float4*>(C)[(size_t)k * 2 + 1];
                c[0] = ca.x; c[1] = ca.y; c[2] = ca.z; c[3] = ca.w;
                c[4] = cb.x; c[5] = cb.y; c[6] = cb.z; c[7] = cb.w;
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t) c[t] = t < d ? C[(size_t)k * d + t] : 0.f;
            }
            float e = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) e = fmaf(bw[t], -2.f * c[t], e);
#pragma unroll
            for (int t = 0; t < 8; ++t) e = fmaf(om[t], c[t] * c[t], e);
            const float v = ldexpf(e, shift_s);
            if (v < v1) {
                v2 = v1;
                v1 = v;
                kb = k;
            } else {
                v2 = fminf(v2, v);
            }
        }
    }
    b1 = v1;
    const float sec = fminf(b2, v2);

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
    const float eb = 48.f * u * (9.f * S_sc + 4.f * fmaxf(gb, -S_sc)) + 1.f;
    const float es = 48.f * u * (9.f * S_sc + 4.f * fmaxf(gs, -S_sc)) + 1.f;
    // all weights zero: every D is exactly 0 and the lowest index wins
    if (allzero) gk = 0;
    const bool certified = allzero || ((gs - gb) > (eb + es) && gk < K && !bad);

    const bool writer = writer_ok && half == 0;
    if (writer && certified) {
        idx[s] = (uint16_t)gk;
        if (dist) {
            double omd[8];
            float xs[8];
            exact_weights(hcol, rho, mask, s, nb, d, omd);
            for (int t = 0; t < d; ++t) xs[t] = X[s * d + t];
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

// Workgroup = kWaves wavefronts x 32 sub-vectors (consecutive ones, or the
// next 256 entries of a list); lane l of a
// wavefront works on sub-vector (l & 31) of its 32: the lanes of the lower
// half supply the scaled omega*x parts (MFMA k-slots 0-7), those of the
// upper half the scaled omega parts (k-slots 8-15).  The split codebook
// (padded to whole chunks) streams through LDS in chunks of kChunkTiles*32
// centroids, double buffered: the next chunk is fetched into registers
// while the current one is searched, so there is one barrier per chunk.
// Within a wave the tiles are software pipelined: tile t's MFMAs are issued
// with tile t-1's argmin updates between them (two accumulators alternate).
// SLOT selects per-slot tracking (short codebooks) over per-tile tracking
// with the best tile formed again at the end (long codebooks).
template <bool SLOT>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(5, 8))) void k_assign_h16(
    const float* __restrict__ X, const float* __restrict__ hcol, const float* __restrict__ rho,
    const uint8_t* __restrict__ mask, int64_t n_sub, int64_t nb, int d, const uint4* __restrict__ P,
    const float* __restrict__ cmax, const float* __restrict__ C, int K, int nchunks,
    const int* __restrict__ list, const int* __restrict__ list_count,
    uint16_t* __restrict__ idx, float* __restrict__ dist, int* __restrict__ flag_count, int* __restrict__ flag_list)
{
    constexpr int kChunkVec = kChunkTiles * 128;                 // uint4 per chunk
    static_assert(kChunkTiles % 2 == 0, "tiles are processed in pairs");
    static_assert(kChunkVec == 2 * kWaves * 64, "two uint4 per thread per chunk");
    __shared__ uint4 lds[2][kChunkVec];

    // without a list: sub-vectors 0 .. n_sub-1; with one: list[0 .. *list_count-1]
    const int64_t count = list ? (int64_t)*list_count : n_sub;
    if ((int64_t)blockIdx.x * kSubPerBlock >= count) return;     // whole workgroup idle
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int64_t w0 = ((int64_t)blockIdx.x * kWaves + wave) * kSubPerWave;
    const bool active = w0 < count;                               // wave-uniform
    const int64_t q = w0 + (lane & 31);
    const bool valid = q < count;
    const int64_t s = valid ? (list ? (int64_t)list[q] : q) : 0;

    // ---- the sub-vector's weights, scaled split B operand, S -----------
    const bool vecX = d == 8 && ((reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(hcol)) & 15u) == 0;
    h16x8 bh, bl;
    float S_sc;
    int shift_s;   // S_sc = S * 2^shift_s: the sub-vector's scale alpha*beta
    {
        float raw[8];
        float S = 0.f;
        float xs[8], ws_[8];
        load_sub(X, hcol, mask, s, nb, d, valid, vecX, xs, ws_);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float xv = xs[t], w = ws_[t];
            S += w * xv * xv;
            // lower half: omega*x (scale alpha*beta); upper half: omega
            // (scale alpha*beta2*(beta/beta2))
            raw[t] = half ? w : w * xv;
        }
        int e1, e2;
        cb_exponents(*cmax, e1, e2);
        float mx = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) mx = fmaxf(mx, fabsf(raw[t]));
        // alpha from the larger of the two halves
        const int rel = half ? (e2 - e1) : 0;
        int ex = -100000;
        if (mx > 0.f) {
            frexpf(mx, &ex);
            ex += rel;
        }
        int en = max(ex, __shfl_xor(ex, 32));
        if (en < -50000) en = 0;                                  // all weights zero
        const int shift = (15 - en) + rel;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            _Float16 h, l;
            split_h16(ldexpf(raw[t], shift), h, l);
            bh[t] = h;
            bl[t] = l;
        }
        shift_s = (15 - en) + (15 - e1);
        S_sc = ldexpf(S, shift_s);
    }

    float b1 = __builtin_inff(), b2 = __builtin_inff();
    int kt1 = 0;

    uint4 pre0 = P[threadIdx.x];
    uint4 pre1 = P[threadIdx.x + kWaves * 64];
    lds[0][threadIdx.x] = pre0;
    lds[0][threadIdx.x + kWaves * 64] = pre1;
    __syncthreads();

    // accB holds the pending tile; +inf values leave the slots unchanged
    f32x16 accA, accB;
    for (int j = 0; j < 16; ++j) accB[j] = __builtin_inff();
    int ktB = 0;
    const int a_off = half * 32 + (lane & 31);
    for (int c = 0; c < nchunks; ++c) {
        if (c + 1 < nchunks) {
            const uint4* src = P + (size_t)(c + 1) * kChunkVec;
            pre0 = src[threadIdx.x];
            pre1 = src[threadIdx.x + kWaves * 64];
        }
        if (active) {
            const uint4* L = lds[c & 1] + a_off;
            const int kt0 = c * kChunkTiles;
#pragma unroll 1
            for (int tt = 0; tt < kChunkTiles; tt += 2) {
                const uint4* A0 = L + tt * 128;
                const uint4* A1 = A0 + 128;
                const h16x8 ah0 = __builtin_bit_cast(h16x8, A0[0]);
                const h16x8 al0 = __builtin_bit_cast(h16x8, A0[64]);
                accA = tile_h16<SLOT>(ah0, al0, bh, bl, accB, ktB, b1, b2, kt1);
                const h16x8 ah1 = __builtin_bit_cast(h16x8, A1[0]);
                const h16x8 al1 = __builtin_bit_cast(h16x8, A1[64]);
                accB = tile_h16<SLOT>(ah1, al1, bh, bl, accA, kt0 + tt, b1, b2, kt1);
                ktB = kt0 + tt + 1;
            }
        }
        if (c + 1 < nchunks) {
            lds[(c + 1) & 1][threadIdx.x] = pre0;
            lds[(c + 1) & 1][threadIdx.x + kWaves * 64] = pre1;
        }
        __syncthreads();
    }
    if (!active) return;
    track<SLOT>(accB, ktB, b1, b2, kt1);

    search_epilogue<SLOT>(X, hcol, rho, mask, nb, d, C, K, s, valid, valid, false, false, lane, half, b1, b2,
                          kt1, S_sc, shift_s, idx, dist, flag_count, flag_list);
}

// Sub-vectors that share one weight vector: workgroup = column block b x
// 256*NS consecutive rows (wavefront w: NS sets of 32 rows, set u holding rows
// (rb*8 + w)*32*NS + u*32 + (l & 31)), taken with the block's majority mask
// byte.  Every A operand read from LDS feeds the MFMAs of all NS sets, so the
// LDS traffic per MFMA falls as 1/NS.  Their common weights make
// sum_t omega_t c_t^2 a per-centroid bias.  The workgroup forms it once per
// chunk in float64 (rounded once to fp32), scales it by 2^sb and splits it
// into two fp16 parts that enter the second MFMA through two k-slots against
// a power-of-two gamma on the B side.  A tile then takes two MFMAs:
//   1: lower half al(-2 beta c) . bh(alpha omega x), upper half ah(-2 beta c) . bl(alpha omega x)
//   2: lower half ah(-2 beta c) . bh(alpha omega x), upper half [bias_hi, bias_lo] . [gamma, gamma]
// with gamma = alpha * beta * 2^-sb.  alpha is capped so that gamma <= 2^15.
// A lane whose gamma would fall below 2^-24 is sent to the exact re-search.
// The general form's error bound holds: the bias is within 1.25u of
// sum omega c*c, and the last MFMA adds 10 products to a small accumulator.
// Lanes whose own mask byte differs from the block's are computed but not
// written: they are in the list of the general kernel.
template <bool SLOT, int NS>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(NS == 1 ? 4 : (NS == 2 ? 3 : 2), 8))) void k_assign_h16s(
    const float* __restrict__ X, const float* __restrict__ hcol, const float* __restrict__ rho,
    const uint8_t* __restrict__ mask, const uint8_t* __restrict__ pattern, int64_t M, int64_t nb, int d,
    const uint4* __restrict__ P, const float* __restrict__ cmax, const float* __restrict__ C, int K, int nchunks,
    uint16_t* __restrict__ idx, float* __restrict__ dist, int* __restrict__ flag_count, int* __restrict__ flag_list)
{
    constexpr int kRowVec = kChunkTiles * 96;    // uint4 per chunk: rows (lo, hi, bias) of 32 per tile
    static_assert(kChunkTiles * 64 == kWaves * 64, "one cross-term uint4 per thread per chunk");
    static_assert(kChunkTiles % 2 == 0, "tiles are processed in pairs");
    __shared__ uint4 lds[2][kRowVec];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int64_t rb = (int64_t)blockIdx.x / nb;
    const int64_t b = (int64_t)blockIdx.x - rb * nb;
    // NS sets of 32 rows per wave: set u holds rows w0 + u*32 + (l & 31)
    const int64_t w0 = (rb * kWaves + wave) * (int64_t)(kSubPerWave * NS);
    const bool active = w0 < M;                                   // wave-uniform
    const unsigned pat = pattern ? pattern[b] : 0u;
    // Row i of set u, its sub-vector id s and whether its weights are the
    // block's; formed before the main loop and again after it (r is passed
    // through an empty asm so the second forming is not merged with the
    // first: keeping these per-set values alive across the loop would spill).
    auto row_of = [&](int u, int r, int64_t& s, bool& valid, bool& owner) {
        const int64_t i = w0 + u * kSubPerWave + r;
        valid = i < M;
        s = valid ? i * nb + b : 0;
        const unsigned mb = (valid && mask) ? mask[s] : 0u;
        owner = valid && mb == pat;
    };

    // the block's weights (its majority pattern), the same in every lane:
    // kept in scalar registers
    float om[8];
    float wsum = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const float w = (t < d && !((pat >> t) & 1u)) ? hcol[b * d + t] : 0.f;
        om[t] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, w)));
        wsum += om[t];
    }
    int e1, e2;
    cb_exponents(*cmax, e1, e2);
    // bias scale: every bias_k <= sum_t omega_t * max c^2 (margin for roundings)
    const float cm = *cmax;
    const float bmax = wsum * (cm * cm) * 1.0001f;
    int eb = 0;
    if (bmax > 0.f) frexpf(bmax, &eb);
    const int sb = 15 - eb;                   // bias * 2^sb < 2^15

    // The sub-vector's scaled split B operands, its scaled energy S_sc, its
    // scale exponent and whether gamma underflows.
    auto prep = [&](int64_t s, bool valid, h16x8& bA, h16x8& bB, float& S_sc, int& shift_s, bool& bad) {
        float raw[8];
        float S = 0.f, mx = 0.f;
        float xs[8];
        if (valid && d == 8 && (reinterpret_cast<uintptr_t>(X) & 15u) == 0) {
            const float4 x0 = reinterpret_cast<const float4*>(X)[(size_t)s * 2];
            const float4 x1 = reinterpret_cast<const float4*>(X)[(size_t)s * 2 + 1];
            xs[0] = x0.x; xs[1] = x0.y; xs[2] = x0.z; xs[3] = x0.w;
            xs[4] = x1.x; xs[5] = x1.y; xs[6] = x1.z; xs[7] = x1.w;
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) xs[t] = (valid && t < d) ? X[s * d + t] : 0.f;
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float xv = xs[t];
            S += om[t] * xv * xv;
            raw[t] = om[t] * xv;
            mx = fmaxf(mx, fabsf(raw[t]));
        }
        int ex = 0;
        if (mx > 0.f) frexpf(mx, &ex);
        const int cap = sb + e1;                                  // keeps gamma <= 2^15
        const int sh = mx > 0.f ? min(15 - ex, cap) : cap;
        const int gexp = sh + (15 - e1) - sb;
        bad = gexp < -24;
        h16x8 bh, bl;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            _Float16 h, l;
            split_h16(ldexpf(raw[t], sh), h, l);
            bh[t] = h;
            bl[t] = l;
        }
        h16x8 gv = {};
        const _Float16 g = (_Float16)ldexpf(1.f, max(gexp, -24));
        gv[0] = g;
        gv[1] = g;
        bA = half ? bl : bh;
        bB = half ? gv : bh;
        shift_s = sh + (15 - e1);
        S_sc = ldexpf(S, shift_s);
    };
    h16x8 bA[NS], bB[NS];    // B operands of the two MFMAs (per half), per set
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        int64_t s;
        bool valid, owner, bad;
        float S_sc;
        int shift_s;
        row_of(u, lane & 31, s, valid, owner);
        prep(s, valid, bA[u], bB[u], S_sc, shift_s, bad);
    }

    // chunk staging: thread q copies one cross-term uint4 (tile q/64, row
    // (q/32)&1: 0 = lo, 1 = hi, position q&31); threads q < 256 form the bias
    // part of centroid q of the chunk
    const int ct = threadIdx.x >> 6, crow = (threadIdx.x >> 5) & 1, cpos = threadIdx.x & 31;
    const bool vecC = d == 8 && (reinterpret_cast<uintptr_t>(C) & 15u) == 0;
    auto load_cross = [&](int c) -> uint4 {
        return P[(size_t)(c * kChunkTiles + ct) * 128 + (crow == 0 ? 64 : 0) + cpos];
    };
    auto load_row = [&](int c, float4& r0, float4& r1) {
        r0 = make_float4(0.f, 0.f, 0.f, 0.f);
        r1 = r0;
        const int k = c * kChunkTiles * kTile + (int)threadIdx.x;
        if (threadIdx.x >= kChunkTiles * kTile || k >= K) return;
        if (vecC) {
            r0 = reinterpret_cast<const float4*>(C)[(size_t)k * 2];
            r1 = reinterpret_cast<const float4*>(C)[(size_t)k * 2 + 1];
        } else {
            float v[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) v[t] = t < d ? C[(size_t)k * d + t] : 0.f;
            r0 = make_float4(v[0], v[1], v[2], v[3]);
            r1 = make_float4(v[4], v[5], v[6], v[7]);
        }
    };
    auto store_chunk = [&](int buf, int c, const uint4& cross, const float4& r0, const float4& r1) {
        lds[buf][ct * 96 + crow * 32 + cpos] = cross;
        if (threadIdx.x < kChunkTiles * kTile) {
            const int k = c * kChunkTiles * kTile + (int)threadIdx.x;
            float a;
            if (k < K) {
                const double cv[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
                double acc = 0.0;
#pragma unroll
                for (int t = 0; t < 8; ++t) acc = acc + (double)om[t] * (cv[t] * cv[t]);
                a = ldexpf((float)acc, sb);
            } else {
                a = kPadSq;
            }
            _Float16 h, l;
            split_h16(a, h, l);
            h16x8 v = {};
            v[0] = h;
            v[1] = l;
            const int tt = threadIdx.x >> 5, m = threadIdx.x & 31;
            lds[buf][tt * 96 + 64 + m] = __builtin_bit_cast(uint4, v);
        }
    };

    float b1[NS], b2[NS];
    int kt1[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        b1[u] = __builtin_inff();
        b2[u] = __builtin_inff();
        kt1[u] = 0;
    }
    uint4 pre = load_cross(0);
    float4 r0, r1;
    load_row(0, r0, r1);
    store_chunk(0, 0, pre, r0, r1);
    __syncthreads();

    // each set's A operands are read from LDS once per tile and used by the
    // MFMAs of every set
    f32x16 accA[NS], accB[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u)
        for (int j = 0; j < 16; ++j) accB[u][j] = __builtin_inff();
    int ktB = 0;
    const int a_off = half * 32 + (lane & 31);
    for (int c = 0; c < nchunks; ++c) {
        if (c + 1 < nchunks) {
            pre = load_cross(c + 1);
            load_row(c + 1, r0, r1);
        }
        if (active) {
            const uint4* L = lds[c & 1] + a_off;
            const int kt0 = c * kChunkTiles;
#pragma unroll 1
            for (int tt = 0; tt < kChunkTiles; tt += 2) {
                const uint4* A0 = L + tt * 96;
                const uint4* A1 = A0 + 96;
                const h16x8 p0 = __builtin_bit_cast(h16x8, A0[0]);
                const h16x8 q0 = __builtin_bit_cast(h16x8, A0[32]);
#pragma unroll
                for (int u = 0; u < NS; ++u)
                    accA[u] = tile2_h16<SLOT>(p0, q0, bA[u], bB[u], accB[u], ktB, b1[u], b2[u], kt1[u]);
                const h16x8 p1 = __builtin_bit_cast(h16x8, A1[0]);
                const h16x8 q1 = __builtin_bit_cast(h16x8, A1[32]);
#pragma unroll
                for (int u = 0; u < NS; ++u)
                    accB[u] = tile2_h16<SLOT>(p1, q1, bA[u], bB[u], accA[u], kt0 + tt, b1[u], b2[u], kt1[u]);
                ktB = kt0 + tt + 1;
            }
        }
        if (c + 1 < nchunks) store_chunk((c + 1) & 1, c + 1, pre, r0, r1);
        __syncthreads();
    }
    if (!active) return;
#pragma unroll
    for (int u = 0; u < NS; ++u) track<SLOT>(accB[u], ktB, b1[u], b2[u], kt1[u]);
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        int r = lane & 31;
        asm volatile("" : "+v"(r));
        int64_t s;
        bool valid, owner, bad;
        float S_sc;
        int shift_s;
        h16x8 ua, ub;
        row_of(u, r, s, valid, owner);
        prep(s, valid, ua, ub, S_sc, shift_s, bad);
        search_epilogue<SLOT>(X, hcol, rho, mask, nb, d, C, K, s, valid, owner, bad, wsum == 0.f, lane, half, b1[u],
                              b2[u], kt1[u], S_sc, shift_s, idx, dist, flag_count, flag_list);
    }
}

// Exact re-search of the flagged sub-vectors: one wavefront per flagged
// sub-vector (grid-stride), its lanes striding over the codebook.  For each
// centroid the float32 expanded form e~ (a fused multiply-add chain over the
// 16 terms: the search's rounding bound applies) is formed; a lane keeps a
// running approximate minimum b~, and a centroid whose interval e~ - err(e~)
// reaches b~ + err(b~) is evaluated in float64 in the direct form, exactly
// as a plain float64 evaluation rounds.  Every exact minimizer lies in the
// final window, which is contained in the evaluated set, so the
// lexicographic (D, k) minimum over the wavefront is the exact argmin (ties
// to the lowest index).  Dimensions >= d carry weight 0 and add exact zeros.
__global__ __launch_bounds__(256) void k_assign_exact(
    const float* __restrict__ X, const float* __restrict__ hcol, const float* __restrict__ rho,
    const uint8_t* __restrict__ mask, int64_t nb, int d, const float* __restrict__ C, int K,
    const int* __restrict__ flag_count, const int* __restrict__ flag_list,
    uint16_t* __restrict__ idx, float* __restrict__ dist, int vecC)
{
    const int n = *flag_count;
    const int lane = threadIdx.x & 63;
    const float u = 5.9604644775390625e-8f;
    const int waves = gridDim.x * (blockDim.x >> 6);
    for (int f = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); f < n; f += waves) {
        const int64_t s = flag_list[f];
        const int64_t i = s / nb, b = s - i * nb;
        const unsigned mb = mask ? mask[s] : 0u;
        const double rr = rho ? (double)rho[i] : 1.0;
        float x[8], om[8], bw2[8];
        double w64[8];
        float S = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const bool on = t < d;
            x[t] = on ? X[s * d + t] : 0.f;
            om[t] = (on && !((mb >> t) & 1u)) ? hcol[b * d + t] : 0.f;
            bw2[t] = -2.f * (om[t] * x[t]);   // exact: fma(-2 bw, c, e) == fma(bw, -2 c, e)
            S += om[t] * x[t] * x[t];
            double w = (double)om[t];
            if (rho) w = w * rr;
            w64[t] = w;
        }
        // filter bound err(e) = 32u (9 S + 4 max(e, -S)) + 1e-35 = A + B max(e, -S)
        const float A = 32.f * u * 9.f * S + 1.0e-35f;
        const float B = 128.f * u;
        float thr = __builtin_inff();
        double dbest = __builtin_inf();
        int arg = K;
        auto load_c = [&](int k, float* c) {
            if (vecC) {   // d == 8 and a 16-byte aligned codebook
                const float4 ca = reinterpret_cast<const float4*>(C)[(size_t)k * 2];
                const float4 cb = reinterpret_cast<const float4*>(C)[(size_t)k * 2 + 1];
                c[0] = ca.x; c[1] = ca.y; c[2] = ca.z; c[3] = ca.w;
                c[4] = cb.x; c[5] = cb.y; c[6] = cb.z; c[7] = cb.w;
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t) c[t] = t < d ? C[(size_t)k * d + t] : 0.f;
            }
        };
        auto visit = [&](int k, const float* c) {
            float e = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) e = fmaf(bw2[t], c[t], e);
#pragma unroll
            for (int t = 0; t < 8; ++t) e = fmaf(om[t], c[t] * c[t], e);
            const float mm = fmaxf(e, -S);
            if (fmaf(-B, mm, e) - A <= thr) {
                thr = fminf(thr, e + fmaf(B, mm, A));
                double acc = 0.0;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const double diff = (double)x[t] - (double)c[t];
                    const double sq = diff * diff;
                    acc = acc + w64[t] * sq;
                }
                if (acc < dbest) { dbest = acc; arg = k; }
            }
        };
        // a lane's centroids k = lane, lane + 64, ... in increasing order; the
        // rows of four steps are loaded before any of them is visited
        int k = lane;
        for (; k + 192 < K; k += 256) {
            float c0[8], c1[8], c2[8], c3[8];
            load_c(k, c0);
            load_c(k + 64, c1);
            load_c(k + 128, c2);
            load_c(k + 192, c3);
            visit(k, c0);
            visit(k + 64, c1);
            visit(k + 128, c2);
            visit(k + 192, c3);
        }
        for (; k < K; k += 64) {
            float c[8];
            load_c(k, c);
            visit(k, c);
        }
        for (int off = 32; off > 0; off >>= 1) {
            const double od = __shfl_xor(dbest, off);
            const int ok = __shfl_xor(arg, off);
            if (od < dbest || (od == dbest && ok < arg)) { dbest = od; arg = ok; }
        }
        if (lane == 0) {
            idx[s] = (uint16_t)arg;
            if (dist) dist[s] = (float)dbest;
        }
    }
}

}  // namespace

// Centroids per LDS chunk; the split codebook is padded to whole chunks.
constexpr int kChunkK = kChunkTiles * kTile;
// Row sets of 32 per wave in the shared-weight search, and rows per workgroup.
constexpr int kSharedSets = 4;
constexpr int kSharedRows = kSubPerBlock * kSharedSets;

inline int padded_K(int K) { return (K + kChunkK - 1) / kChunkK * kChunkK; }

size_t ws_assign(int64_t n_sub, int K)
{
    // split codebook (64 bytes per centroid), flag counter, flag list, max |c|,
    // partial maxima, dirty counter, dirty list, block patterns (at most n_sub
    // column blocks)
    return align_up((size_t)padded_K(K) * 64) + align_up(sizeof(int)) + align_up((size_t)n_sub * sizeof(int)) +
           align_up(sizeof(float)) + align_up(sizeof(float) * kMaxBlocks) + align_up(sizeof(int)) +
           align_up((size_t)n_sub * sizeof(int)) + align_up((size_t)n_sub);
}

// Enqueues the assignment; arguments already validated by the caller.
vq_status assign_launch(const float* X, const float* hcol, const float* rho, const uint8_t* mask,
                        int64_t M, int64_t N, int d, const float* C, int K,
                        uint16_t* idx, float* dist, void* ws, size_t ws_bytes, hipStream_t st)
{
    const int64_t n_sub = M * N / d;
    const int64_t nb = N / d;
    const int Kpad = padded_K(K);
    Carver cv(ws, ws_bytes);
    uint4* P = cv.take<uint4>((size_t)Kpad * 4);
    int* flag_count = cv.take<int>(1);
    int* flag_list = cv.take<int>((size_t)n_sub);
    float* cmax = cv.take<float>(1);
    float* part = cv.take<float>(kMaxBlocks);
    int* dirty_count = cv.take<int>(1);
    int* dirty_list = cv.take<int>((size_t)n_sub);
    uint8_t* pattern = cv.take<uint8_t>((size_t)nb);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_assign: workspace too small");
    if (n_sub > (int64_t)INT32_MAX) return fail(VQ_ERR_UNSUPPORTED, "vq_assign: more than 2^31 sub-vectors");
    const int64_t shared_groups = (M + kSharedRows - 1) / kSharedRows * nb;
    if (shared_groups > (int64_t)UINT32_MAX) return fail(VQ_ERR_UNSUPPORTED, "vq_assign: grid too large");

    TimedRegion tr_all("assign", K, st);
    const int nparts = (int)std::min<int64_t>(kMaxBlocks, ((int64_t)K * d + 255) / 256);
    hipLaunchKernelGGL(k_cb_absmax_part, dim3(nparts), dim3(256), 0, st, C, (int64_t)K * d, part);
    VQ_LAUNCHED("k_cb_absmax_part");
    hipLaunchKernelGGL(k_cb_absmax_final, dim3(1), dim3(256), 0, st, part, nparts, cmax, flag_count, dirty_count);
    VQ_LAUNCHED("k_cb_absmax_final");
    hipLaunchKernelGGL(k_cb_prep16, dim3(grid_for(Kpad, 256)), dim3(256), 0, st, C, K, d, Kpad, cmax, P);
    VQ_LAUNCHED("k_cb_prep16");
    {
        TimedRegion tr("assign_search", K, st);
        const int nch = Kpad / kChunkK;
        const bool slot = nch <= kSlotChunks;
        if (slot) {
            // short codebooks: one pass of the general form (the block
            // classification would cost more than the shared form saves)
            hipLaunchKernelGGL(k_assign_h16<true>, dim3(grid_for(n_sub, kSubPerBlock)), dim3(kWaves * 64), 0, st, X,
                               hcol, rho, mask, n_sub, nb, d, P, cmax, C, K, nch, nullptr, nullptr, idx, dist,
                               flag_count, flag_list);
            VQ_LAUNCHED("k_assign_h16");
        } else {
        if (mask) {
            hipLaunchKernelGGL(k_block_pattern, dim3((unsigned)nb), dim3(256), 0, st, mask, M, nb, pattern);
            VQ_LAUNCHED("k_block_pattern");
            hipLaunchKernelGGL(k_dirty, dim3(grid_for(n_sub, 4096)), dim3(1024), 0, st, mask, pattern, n_sub,
                               (uint32_t)nb, dirty_count, dirty_list);
            VQ_LAUNCHED("k_dirty");
        }
        // sub-vectors with their block's weights: two MFMAs per tile
        hipLaunchKernelGGL((k_assign_h16s<false, kSharedSets>), dim3((unsigned)shared_groups), dim3(kWaves * 64), 0, st, X, hcol,
                           rho, mask, mask ? pattern : nullptr, M, nb, d, P, cmax, C, K, nch, idx, dist, flag_count,
                           flag_list);
        VQ_LAUNCHED("k_assign_h16s");
        // the rest, each with its own weights: three MFMAs per tile
        if (mask) {
            hipLaunchKernelGGL(k_assign_h16<false>, dim3(grid_for(n_sub, kSubPerBlock)), dim3(kWaves * 64), 0, st, X,
                               hcol, rho, mask, n_sub, nb, d, P, cmax, C, K, nch, dirty_list, dirty_count, idx, dist,
                               flag_count, flag_list);
            VQ_LAUNCHED("k_assign_h16");
        }
        }
    }
    const unsigned gx = (unsigned)std::min<int64_t>((n_sub + 3) / 4, kExactBlocks);
    const int vecC = (d == 8 && (reinterpret_cast<uintptr_t>(C) & 15u) == 0) ? 1 : 0;
    hipLaunchKernelGGL(k_assign_exact, dim3(gx), dim3(256), 0, st, X, hcol, rho, mask, nb, d, C, K,
                       flag_count, flag_list, idx, dist, vecC);
    VQ_LAUNCHED("k_assign_exact");
    return VQ_OK;
}

// Number of sub-vectors the last search sent to the exact path (diagnostics).
vq_status assign_flag_count(void* ws, size_t ws_bytes, int64_t n_sub, int K, int* out, hipStream_t st)
{
    Carver cv(ws, ws_bytes);
    cv.take<uint4>((size_t)padded_K(K) * 4);
    int* flag_count = cv.take<int>(1);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "workspace too small");
    VQ_HIP(hipMemcpyAsync(out, flag_count, sizeof(int), hipMemcpyDeviceToHost, st));
    VQ_HIP(hipStreamSynchronize(st));
    (void)n_sub;
    return VQ_OK;
}

}  // namespace vq
