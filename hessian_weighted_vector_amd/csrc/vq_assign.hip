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
#include <mutex>
#include <vector>

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
constexpr int kCminChunks = 8;            // chunks per workgroup of the chunk-minimum pass
constexpr int kCminCap = 32768;           // flagged sub-vectors the chunk path takes at most
constexpr int kCminListBlocks = 64;       // list blocks of the chunk-minimum grid (grid-stride)
constexpr int kBlockPatterns = 4;         // shared weight patterns per column block (bias pairs in k-slots 8-15)
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

// Short codebooks: the tile tracking above, plus the 16 values of the lane's
// best tile kept in registers (a select per value, no branch).  At the end
// park_resolve finds the best's slot in that tile (the first of equal
// values: slot order is centroid order within the lane, so the lower index)
// and folds the tile's own second best into b2; pos becomes kt*16 + slot.
__device__ __forceinline__ void park_track(const f32x16& a, int kt, float& b1, float& b2, int& kt1,
                                           float (&pk)[16])
{
    const float tm = tile_min(a);
    b2 = __builtin_amdgcn_fmed3f(b1, tm, b2);
    const bool lt = tm < b1;
    b1 = lt ? tm : b1;
    kt1 = lt ? kt : kt1;
#pragma unroll
    for (int j = 0; j < 16; ++j) pk[j] = lt ? a[j] : pk[j];
}

__device__ __forceinline__ void park_resolve(const float (&pk)[16], float b1, float& b2, int& pos)
{
    int jj = 0, ties = 0;
    float t2 = __builtin_inff();                          // smallest value above the best
#pragma unroll
    for (int j = 15; j >= 0; --j) {
        if (pk[j] == b1) {
            jj = j;
            ++ties;
        } else {
            t2 = fminf(t2, pk[j]);
        }
    }
    b2 = fminf(b2, ties > 1 ? b1 : t2);
    pos = pos * 16 + jj;
}

template <bool SLOT>
__device__ __forceinline__ void track(const f32x16& a, int kt, float& b1, float& b2, int& pos, float (&pk)[16])
{
    if (SLOT)
        park_track(a, kt, b1, b2, pos, pk);
    else
        tile_track(a, kt, b1, b2, pos);
}

// One 32x32 tile: three chained MFMAs (lo*hi, hi*lo, then hi*hi), with the
// previous tile's tracking update between them.
template <bool SLOT>
__device__ __forceinline__ f32x16 tile_h16(const h16x8 ah, const h16x8 al, const h16x8 bh, const h16x8 bl,
                                           const f32x16& prev, int ktp, float& b1, float& b2, int& pos,
                                           float (&pk)[16])
{
    f32x16 acc = {};
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, acc, 0, 0, 0);
    track<SLOT>(prev, ktp, b1, b2, pos, pk);
#pragma unroll
    for (int g = 0; g < 3; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // four VALU
    }
    return acc;
}

// The (up to) four most frequent mask bytes of each column block, most
// frequent first and the lower byte first among equal counts, packed one
// byte each into a 32-bit word; a block with fewer distinct bytes repeats its
// first in the remaining slots.  Sub-vectors with one of these bytes share
// that byte's weights with the rest of its class.
__global__ __launch_bounds__(256) void k_block_pattern(const uint8_t* __restrict__ mask, int64_t M, int64_t nb,
                                                       uint32_t* __restrict__ pattern)
{
    __shared__ int cnt[256];
    __shared__ int best_c[256], best_p[256];
    cnt[threadIdx.x] = 0;
    __syncthreads();
    const int64_t b = blockIdx.x;
    for (int64_t i = threadIdx.x; i < M; i += 256) atomicAdd(&cnt[mask[i * nb + b]], 1);
    __syncthreads();
    uint32_t word = 0;
    for (int q = 0; q < kBlockPatterns; ++q) {
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
        const int c = best_c[0], p = best_p[0];
        // slot 0 always has a count >= 1 (M >= 1); an empty slot repeats it
        word |= (uint32_t)(c > 0 ? p : (int)(word & 0xFFu)) << (8 * q);
        __syncthreads();
        if (threadIdx.x == 0) cnt[p] = -1;
        __syncthreads();
    }
    if (threadIdx.x == 0) pattern[b] = word;
}

// Slot (0-3) of mask byte mb among a block's pattern word, or -1.
__device__ __forceinline__ int pattern_slot(uint32_t word, unsigned mb)
{
    int q = -1;
#pragma unroll
    for (int t = kBlockPatterns - 1; t >= 0; --t)
        if (((word >> (8 * t)) & 0xFFu) == mb) q = t;
    return q;
}

// Sub-vectors whose mask byte is none of their block's patterns are listed
// for the general kernel: wavefront ballots, a workgroup prefix in LDS and
// one integer atomic per workgroup (the order of the list does not affect
// any result).
__global__ __launch_bounds__(1024) void k_dirty(const uint8_t* __restrict__ mask, const uint32_t* __restrict__ pattern,
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
        if (s < n_sub) take[r] = pattern_slot(pattern[(uint32_t)(s % nb)], mask[s]) < 0;
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
    static_assert(!SLOT, "the shared-weight form tracks tiles");
    tile_track(prev, ktp, b1, b2, pos);
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
// SLOT (short codebooks) keeps the best tile's values in registers and finds
// the best's slot at the end; otherwise (long codebooks) the best tile is
// formed again at the end.
// The general form's B operand of one sub-vector: the lanes of the lower
// half hold the scaled omega*x parts (MFMA k-slots 0-7), those of the upper
// half the scaled omega parts (k-slots 8-15), each split into two fp16
// parts; S_sc = S * 2^shift_s is the sub-vector's sum omega x^2 at the same
// scale (the rounding bound's S).
__device__ __forceinline__ void general_operand(const float* __restrict__ X, const float* __restrict__ hcol,
                                                const uint8_t* __restrict__ mask, int64_t s, int64_t nb, int d,
                                                bool valid, int half, float cmax, h16x8& bh, h16x8& bl,
                                                float& S_sc, int& shift_s)
{
    const bool vecX = d == 8 && ((reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(hcol)) & 15u) == 0;
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
    cb_exponents(cmax, e1, e2);
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

template <bool SLOT>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(SLOT ? 4 : 5, 8))) void k_assign_h16(
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
    h16x8 bh, bl;
    float S_sc;
    int shift_s;   // S_sc = S * 2^shift_s: the sub-vector's scale alpha*beta
    general_operand(X, hcol, mask, s, nb, d, valid, half, *cmax, bh, bl, S_sc, shift_s);

    float b1 = __builtin_inff(), b2 = __builtin_inff();
    int kt1 = 0;
    float pk[16];                                                // short codebooks: the best tile's values
#pragma unroll
    for (int j = 0; j < 16; ++j) pk[j] = __builtin_inff();

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
                accA = tile_h16<SLOT>(ah0, al0, bh, bl, accB, ktB, b1, b2, kt1, pk);
                const h16x8 ah1 = __builtin_bit_cast(h16x8, A1[0]);
                const h16x8 al1 = __builtin_bit_cast(h16x8, A1[64]);
                accB = tile_h16<SLOT>(ah1, al1, bh, bl, accA, kt0 + tt, b1, b2, kt1, pk);
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
    track<SLOT>(accB, ktB, b1, b2, kt1, pk);
    if (SLOT) park_resolve(pk, b1, b2, kt1);

    search_epilogue<SLOT>(X, hcol, rho, mask, nb, d, C, K, s, valid, valid, false, false, lane, half, b1, b2,
                          kt1, S_sc, shift_s, idx, dist, flag_count, flag_list);
}

// Codebooks of one chunk (K <= 256), per-slot tracking: the workgroup stages
// the split codebook in LDS once and then takes groups of kSubPerBlock
// consecutive sub-vectors in turn (grid-stride; wavefront w takes the
// group's w-th 32), each searched as in k_assign_h16.  No barrier follows
// the staging, so the waves of a workgroup drift apart freely and the
// codebook crosses from L2 once per workgroup rather than once per group.
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_assign_h16_one(
    const float* __restrict__ X, const float* __restrict__ hcol, const float* __restrict__ rho,
    const uint8_t* __restrict__ mask, int64_t n_sub, int64_t nb, int d, const uint4* __restrict__ P,
    const float* __restrict__ cmax, const float* __restrict__ C, int K, uint16_t* __restrict__ idx,
    float* __restrict__ dist, int* __restrict__ flag_count, int* __restrict__ flag_list)
{
    constexpr int kChunkVec = kChunkTiles * 128;                 // uint4 per chunk
    static_assert(kChunkVec == 2 * kWaves * 64, "two uint4 per thread per chunk");
    __shared__ uint4 lds[kChunkVec];
    lds[threadIdx.x] = P[threadIdx.x];
    lds[threadIdx.x + kWaves * 64] = P[threadIdx.x + kWaves * 64];
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int a_off = half * 32 + (lane & 31);
    const float cm = *cmax;
    for (int64_t g = blockIdx.x; g * kSubPerBlock < n_sub; g += gridDim.x) {
        const int64_t w0 = (g * kWaves + wave) * kSubPerWave;
        if (w0 >= n_sub) break;                                  // wave-uniform; later groups start further on
        const int64_t q = w0 + (lane & 31);
        const bool valid = q < n_sub;
        const int64_t s = valid ? q : 0;
        h16x8 bh, bl;
        float S_sc;
        int shift_s;
        general_operand(X, hcol, mask, s, nb, d, valid, half, cm, bh, bl, S_sc, shift_s);
        float b1 = __builtin_inff(), b2 = __builtin_inff();
        int kt1 = 0;
        float pk[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) pk[j] = __builtin_inff();
        f32x16 accA, accB;
        for (int j = 0; j < 16; ++j) accB[j] = __builtin_inff();
        int ktB = 0;
        const uint4* L = lds + a_off;
#pragma unroll 1
        for (int tt = 0; tt < kChunkTiles; tt += 2) {
            const uint4* A0 = L + tt * 128;
            const uint4* A1 = A0 + 128;
            const h16x8 ah0 = __builtin_bit_cast(h16x8, A0[0]);
            const h16x8 al0 = __builtin_bit_cast(h16x8, A0[64]);
            accA = tile_h16<true>(ah0, al0, bh, bl, accB, ktB, b1, b2, kt1, pk);
            const h16x8 ah1 = __builtin_bit_cast(h16x8, A1[0]);
            const h16x8 al1 = __builtin_bit_cast(h16x8, A1[64]);
            accB = tile_h16<true>(ah1, al1, bh, bl, accA, tt, b1, b2, kt1, pk);
            ktB = tt + 1;
        }
        track<true>(accB, ktB, b1, b2, kt1, pk);
        park_resolve(pk, b1, b2, kt1);
        search_epilogue<true>(X, hcol, rho, mask, nb, d, C, K, s, valid, valid, false, false, lane, half, b1, b2,
                              kt1, S_sc, shift_s, idx, dist, flag_count, flag_list);
    }
}

// ---- coarse pass of the two-pass search (long codebooks, shared weights) ----
// The coarse score is the shared form's second MFMA alone: hi*hi of the
// cross terms plus the class bias.  With x_t = alpha omega_t x_t and
// c_t = -2 beta c_t (scaled), each fp16 part is within 2^-11 of its value in
// the normal range, so the dropped products (those with a lo part) miss at
// most 2^-10 (1 + 2^-10) sum_t |x_t| |c_t|.  Cauchy-Schwarz in the
// omega-weighted inner product gives sum_t |x_t| |c_t| <= 2 sqrt(S B_k), with
// S = sum_t omega_t x_t^2 and B_k = sum_t omega_t c_kt^2 (the bias), and
// sqrt(B_k) <= sqrt(S) + sqrt(D_k) where D_k = e_k + S is the weighted
// distance itself.  So |e~_k - e_k| <= a (sqrt(S) + sqrt(D_k)) + E0 with
// a = 2^-9 (1 + 2^-10) sqrt(S) and E0 = 48u (11 S + 5 |e~|) + 2: the fp32
// accumulation, fp16's subnormal range (all in scaled units) and the bias,
// which the coarse pass forms in fp32 (within 13u of B_k, and B_k <= 4 S +
// 2 |e~| up to terms of second order).  Solving for sqrt(D_k) with the coarse value D~ = e~ + S gives
// sqrt(D_k) <= (a + sqrt(a^2 + 4 (D~ + a sqrt(S) + E0))) / 2, hence a bound
// Ehat(e~) on |e~ - e| from the coarse value alone.  Its slope is below
// 2^-5, so L(v) = v - Ehat(v) grows with v.
constexpr int kGroupChunks = 4;           // chunks per candidate group of the two-pass search
constexpr int kMaxGroups = 64;            // groups of a 65536-centroid codebook
constexpr int kBucketItems = 4;           // sub-vectors per thread of the candidate bucketing
constexpr int kRefineBlocks = 2048;       // workgroups of the candidate search (grid-stride)

__device__ __forceinline__ float coarse_err(float v, float S, float sqS, float a)
{
    const float u = 5.9604644775390625e-8f;   // 2^-24
    const float E0 = 48.f * u * (11.f * S + 5.f * fabsf(v)) + 2.f;
    const float Dt = fmaxf(v + S, 0.f);
    const float y = 0.5f * (a + sqrtf(a * a + 4.f * (Dt + a * sqS + E0)));
    return 1.001f * (a * (sqS + y) + E0);     // margin for this evaluation's roundings
}

// Running minimum of a tile's 16 values (eight three-way minima).
__device__ __forceinline__ float fold16(const f32x16& a, float m)
{
#pragma unroll
    for (int j = 0; j < 16; j += 2) m = fminf(fminf(m, a[j]), a[j + 1]);
    return m;
}

// Closes group g of one lane pair: the two halves' minima are merged and
// inserted into the three smallest group minima (t1 <= t2 <= t3; their groups
// packed in one word, g1 | g2 << 8 | g3 << 16; the earlier group first among
// equal minima) and the fourth smallest t4.
__device__ __forceinline__ void close_group_packed(float& gm, uint32_t g, float& t1, float& t2, float& t3, float& t4,
                                                   uint32_t& gp)
{
    const float m = fminf(gm, __shfl_xor(gm, 32));
    const bool l1 = m < t1, l2 = m < t2, l3 = m < t3;
    const uint32_t a1 = ((gp << 8) | g) & 0xFFFFFFu;
    const uint32_t a2 = (gp & 0xFFu) | (g << 8) | ((gp << 8) & 0xFF0000u);
    const uint32_t a3 = (gp & 0xFFFFu) | (g << 16);
    gp = l1 ? a1 : (l2 ? a2 : (l3 ? a3 : gp));
    t4 = __builtin_amdgcn_fmed3f(t3, m, t4);
    t3 = __builtin_amdgcn_fmed3f(t2, m, t3);
    t2 = __builtin_amdgcn_fmed3f(t1, m, t2);
    t1 = fminf(t1, m);
    gm = __builtin_inff();
}

// Appends the lanes with take set to a list (one atomic per wavefront; the
// order of the list affects no result).  Every lane of the wavefront calls it.
__device__ __forceinline__ void list_append(bool take, int lane, int64_t s, int* __restrict__ count,
                                            int* __restrict__ list)
{
    const unsigned long long ball = __ballot(take);
    if (ball) {
        int base = 0;
        const int leader = __ffsll((long long)ball) - 1;
        if (lane == leader) base = atomicAdd(count, __popcll(ball));
        base = __shfl(base, leader);
        if (take) list[base + __popcll(ball & ((1ull << lane) - 1ull))] = (int)s;
    }
}

// Sub-vectors whose weights are one of a few per block: workgroup = column
// block b x 256*NS consecutive rows (wavefront w: NS sets of 32 rows, set u
// holding rows (rb*8 + w)*32*NS + u*32 + (l & 31)).  Every A operand read from
// LDS feeds the MFMAs of all NS sets, so the LDS traffic per MFMA falls as
// 1/NS.  The block's pattern word names up to four mask bytes; the sub-vectors
// with pattern q share the weights omega_q, which make sum_t omega_qt c_t^2 a
// per-centroid bias of that class.  The workgroup forms the four biases once
// per chunk in float64 (fused multiply-adds, each sum rounded once to fp32;
// the threads that stage the chunk's centroid rows do it: spreading it over
// every wavefront or into the tile loop measured slower), scales them by 2^sb and
// splits each into two fp16 parts; they fill k-slots 8-15 of the second
// MFMA's A operand, and the B operand of a sub-vector of class q holds a
// power-of-two gamma in slots 8+2q and 9+2q and zeros elsewhere.  A tile then
// takes two MFMAs:
//   1: lower half al(-2 beta c) . bh(alpha omega x), upper half ah(-2 beta c) . bl(alpha omega x)
//   2: lower half ah(-2 beta c) . bh(alpha omega x),
//      upper half [b0_hi, b0_lo, .., b3_hi, b3_lo] . [0, .., gamma, gamma, .., 0]
// with gamma = alpha * beta * 2^-sb.  alpha is capped so that gamma <= 2^15.
// A lane whose gamma would fall below 2^-24 is sent to the exact re-search.
// The general form's error bound holds: the bias is within 1.25u of
// sum omega c*c, and the last MFMA adds 10 nonzero products (the others are
// exact zeros) to a small accumulator.  Lanes whose mask byte is none of the
// block's patterns are computed (with pattern 0) but not written: they are in
// the list of the general kernel.
//
// COARSE: the coarse pass of the two-pass search.  One MFMA per tile (the
// second above) for each of the NS sets, then the sets' folds into the running
// minimum of the current group of kGroupChunks chunks (no accumulator
// ping-pong: the sets' independent MFMAs cover each other's latency, and the
// registers it would take hold twice the sets, so each staged chunk serves
// twice the rows); at each group's end the lane pair's minimum goes into the
// three smallest group minima with their groups and the fourth smallest
// value.  Group g is a candidate when L(m_g) <= U = m_1 + Ehat(m_1)
// (coarse_err); since L grows with m, the candidates are the groups of the
// smallest minima.  Per owned sub-vector: cand[s] = n | g1 << 8 | g2 << 16 |
// g3 << 24 with n the number of candidates (1..3); a sub-vector with a fourth
// candidate goes to the dirty list (the general form over the whole codebook),
// one with all weights zero takes index 0, one whose gamma underflows goes to
// the exact re-search; these and every sub-vector the kernel does not own get
// cand[s] = 0.
template <bool SLOT, int NS, bool COARSE>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(NS == 1 ? 4 : (NS == 2 ? 3 : 2), 8))) void k_assign_h16s(
    const float* __restrict__ X, const float* __restrict__ hcol, const float* __restrict__ rho,
    const uint8_t* __restrict__ mask, const uint32_t* __restrict__ pattern, int64_t M, int64_t nb, int d,
    const uint4* __restrict__ P, const float* __restrict__ cmax, const float* __restrict__ C, int K, int nchunks,
    uint16_t* __restrict__ idx, float* __restrict__ dist, int* __restrict__ flag_count, int* __restrict__ flag_list,
    int* __restrict__ dirty_count, int* __restrict__ dirty_list, uint32_t* __restrict__ cand)
{
    static_assert(kBlockPatterns * 2 == 8, "the four bias pairs fill k-slots 8-15");
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
    const uint32_t pw = (uint32_t)__builtin_amdgcn_readfirstlane((int)(pattern ? pattern[b] : 0u));
    // Row i of set u, its sub-vector id s, whether its weights are one of the
    // block's patterns (owner), its pattern slot q and the mask byte mq its
    // operands are formed with (pattern 0's for a lane that is not an
    // owner); formed before the main loop and again after it (r is passed
    // through an empty asm so the second forming is not merged with the
    // first: keeping these per-set values alive across the loop would spill).
    auto row_of = [&](int u, int r, int64_t& s, bool& valid, bool& owner, int& q, unsigned& mq) {
        const int64_t i = w0 + u * kSubPerWave + r;
        valid = i < M;
        s = valid ? i * nb + b : 0;
        const unsigned mb = (valid && mask) ? mask[s] : 0u;
        const int qs = pattern_slot(pw, mb);
        owner = valid && qs >= 0;
        q = qs >= 0 ? qs : 0;
        mq = (pw >> (8 * q)) & 0xFFu;
    };

    // the block's column weights (no mask), the same in every lane: kept in
    // scalar registers
    float hb[8];
    float wsum = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const float w = t < d ? hcol[b * d + t] : 0.f;
        hb[t] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, w)));
        wsum += hb[t];
    }
    int e1, e2;
    cb_exponents(*cmax, e1, e2);
    // bias scale: every pattern's bias_k <= sum_t h_t * max c^2 (margin for
    // roundings)
    const float cm = *cmax;
    const float bmax = wsum * (cm * cm) * 1.0001f;
    int eb = 0;
    if (bmax > 0.f) frexpf(bmax, &eb);
    const int sb = 15 - eb;                   // bias * 2^sb < 2^15

    // The sub-vector's scaled split B operands, its scaled energy S_sc, its
    // scale exponent and whether gamma underflows.
    auto prep = [&](int64_t s, bool valid, int q, unsigned mq, h16x8& bA, h16x8& bB, float& S_sc, int& shift_s,
                    bool& bad) {
        float om[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) om[t] = ((mq >> t) & 1u) ? 0.f : hb[t];
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
        h16x8 gv;
        const _Float16 g = (_Float16)ldexpf(1.f, max(gexp, -24));
#pragma unroll
        for (int j = 0; j < 8; ++j) gv[j] = (j >> 1) == q ? g : (_Float16)0.f;
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
        int shift_s, q;
        unsigned mq;
        row_of(u, lane & 31, s, valid, owner, q, mq);
        prep(s, valid, q, mq, bA[u], bB[u], S_sc, shift_s, bad);
    }

    // chunk staging: thread q copies one cross-term uint4 (tile q/64, row
    // (q/32)&1: 0 = lo, 1 = hi, position q&31); threads q < 256 form the four
    // biases of centroid q of the chunk
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
            const float cf[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
            double c2[8];
            float c2f[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                if constexpr (COARSE)
                    c2f[t] = cf[t] * cf[t];                       // one rounding
                else
                    c2[t] = (double)cf[t] * (double)cf[t];        // exact
            }
            // one fused multiply-add per term (a masked term adds an exact
            // zero): in float64 with one rounding to fp32 at the end for the
            // certified search; in fp32 for the coarse pass, whose bound
            // carries the sum's rounding (at most 13u of the bias with the
            // squares and the split)
            h16x8 v;
#pragma unroll
            for (int q = 0; q < kBlockPatterns; ++q) {
                const unsigned mq = (pw >> (8 * q)) & 0xFFu;
                float a = kPadSq;
                if (k < K) {
                    if constexpr (COARSE) {
                        float acc = 0.f;
#pragma unroll
                        for (int t = 0; t < 8; ++t) acc = fmaf(((mq >> t) & 1u) ? 0.f : hb[t], c2f[t], acc);
                        a = ldexpf(acc, sb);
                    } else {
                        double acc = 0.0;
#pragma unroll
                        for (int t = 0; t < 8; ++t)
                            acc = __builtin_fma((double)(((mq >> t) & 1u) ? 0.f : hb[t]), c2[t], acc);
                        a = ldexpf((float)acc, sb);
                    }
                }
                _Float16 h, l;
                split_h16(a, h, l);
                v[2 * q] = h;
                v[2 * q + 1] = l;
            }
            const int tt = threadIdx.x >> 5, m = threadIdx.x & 31;
            lds[buf][tt * 96 + 64 + m] = __builtin_bit_cast(uint4, v);
        }
    };

    uint4 pre = load_cross(0);
    float4 r0, r1;
    load_row(0, r0, r1);
    store_chunk(0, 0, pre, r0, r1);
    __syncthreads();
    const int a_off = half * 32 + (lane & 31);

    if constexpr (COARSE) {
        float gmn[NS], t1[NS], t2[NS], t3[NS], t4[NS];
        uint32_t gp[NS];
        f32x16 acc[NS];
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            gmn[u] = t1[u] = t2[u] = t3[u] = t4[u] = __builtin_inff();
            gp[u] = 0;
        }
        for (int c = 0; c < nchunks; ++c) {
            if (c + 1 < nchunks) {
                pre = load_cross(c + 1);
                load_row(c + 1, r0, r1);
            }
            if (active) {
                // per tile: the MFMAs of every set, then their folds (the
                // sets' independent MFMAs cover each other's latency)
                const uint4* L = lds[c & 1] + a_off;
#pragma unroll 1
                for (int t = 0; t < kChunkTiles; ++t) {
                    const h16x8 q = __builtin_bit_cast(h16x8, L[t * 96 + 32]);
#pragma unroll
                    for (int u = 0; u < NS; ++u)
                        acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_f16(q, bB[u], f32x16{}, 0, 0, 0);
#pragma unroll
                    for (int u = 0; u < NS; ++u) gmn[u] = fold16(acc[u], gmn[u]);
                }
                if ((c + 1) % kGroupChunks == 0 || c + 1 == nchunks) {
#pragma unroll
                    for (int u = 0; u < NS; ++u)
                        close_group_packed(gmn[u], (uint32_t)(c / kGroupChunks), t1[u], t2[u], t3[u], t4[u], gp[u]);
                }
            }
            if (c + 1 < nchunks) store_chunk((c + 1) & 1, c + 1, pre, r0, r1);
            __syncthreads();
        }
        if (!active) return;
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            int r = lane & 31;
            asm volatile("" : "+v"(r));
            int64_t s;
            bool valid, owner, bad;
            float S_sc;
            int shift_s, q;
            unsigned mq;
            h16x8 ua, ub;
            row_of(u, r, s, valid, owner, q, mq);
            prep(s, valid, q, mq, ua, ub, S_sc, shift_s, bad);
            bool allz = true;
#pragma unroll
            for (int t = 0; t < 8; ++t) allz = allz && (((mq >> t) & 1u) || hb[t] == 0.f);
            const bool writer = half == 0 && valid;
            bool to_exact = false, to_dirty = false;
            uint32_t cw = 0;
            if (writer && owner) {
                if (allz) {
                    // every weighted distance is exactly 0: the lowest index
                    idx[s] = 0;
                    if (dist) {
                        double omd[8];
                        float xs[8];
                        exact_weights(hcol, rho, mask, s, nb, d, omd);
                        for (int t = 0; t < d; ++t) xs[t] = X[s * d + t];
                        dist[s] = (float)exact_dist(omd, xs, C, d);
                    }
                } else if (bad) {
                    to_exact = true;
                } else {
                    const float sqS = sqrtf(S_sc);
                    const float a = 0x1.004p-9f * sqS;                   // 2^-9 (1 + 2^-10) sqrt(S)
                    const float U = t1[u] + coarse_err(t1[u], S_sc, sqS, a);
                    auto low = [&](float m) {
                        const float mm = fminf(m, 1.0e30f);              // unfilled slots stay far above U
                        return mm - coarse_err(mm, S_sc, sqS, a);
                    };
                    if (low(t4[u]) <= U) {
                        to_dirty = true;
                    } else {
                        const uint32_t n = 1u + (low(t2[u]) <= U ? 1u : 0u) + (low(t3[u]) <= U ? 1u : 0u);
                        cw = n | (gp[u] << 8);
                    }
                }
            }
            if (writer) cand[s] = cw;
            list_append(to_exact, lane, s, flag_count, flag_list);
            list_append(to_dirty, lane, s, dirty_count, dirty_list);
        }
        return;
    }

    float b1[NS], b2[NS];
    int kt1[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        b1[u] = __builtin_inff();
        b2[u] = __builtin_inff();
        kt1[u] = 0;
    }

    // each set's A operands are read from LDS once per tile and used by the
    // MFMAs of every set
    f32x16 accA[NS], accB[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u)
        for (int j = 0; j < 16; ++j) accB[u][j] = __builtin_inff();
    int ktB = 0;
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
    for (int u = 0; u < NS; ++u) tile_track(accB[u], ktB, b1[u], b2[u], kt1[u]);
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        int r = lane & 31;
        asm volatile("" : "+v"(r));
        int64_t s;
        bool valid, owner, bad;
        float S_sc;
        int shift_s, q;
        unsigned mq;
        h16x8 ua, ub;
        row_of(u, r, s, valid, owner, q, mq);
        prep(s, valid, q, mq, ua, ub, S_sc, shift_s, bad);
        search_epilogue<SLOT>(X, hcol, rho, mask, nb, d, C, K, s, valid, owner, bad, wsum == 0.f, lane, half, b1[u],
                              b2[u], kt1[u], S_sc, shift_s, idx, dist, flag_count, flag_list);
    }
}


// ---- candidate groups of the two-pass search ----------------------------
// Entry s * 4 + j of group g's list names candidate j of sub-vector s.

// Fills n ints with v.
__global__ void k_fill_int(int* __restrict__ p, int n, int v)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// Candidates per group: a histogram per workgroup in LDS, then one atomic per
// (workgroup, group).
__global__ __launch_bounds__(1024) void k_cand_count(const uint32_t* __restrict__ cand, int64_t n_sub, int ng,
                                                     int* __restrict__ gcount)
{
    __shared__ int h[kMaxGroups];
    if (threadIdx.x < kMaxGroups) h[threadIdx.x] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kBucketItems; ++r) {
        const int64_t s = ((int64_t)blockIdx.x * kBucketItems + r) * 1024 + threadIdx.x;
        if (s < n_sub) {
            const uint32_t w = cand[s];
            const int n = (int)(w & 3u);
            for (int j = 0; j < n; ++j) atomicAdd(&h[(w >> (8 * (j + 1))) & 0xFFu], 1);
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < ng && h[threadIdx.x]) atomicAdd(&gcount[threadIdx.x], h[threadIdx.x]);
}

// One thread: goff[g] = first list slot of group g, cursor[g] = goff[g],
// gblk[g] = first work item of group g (kSubPerBlock entries per item),
// gblk[ng] = the number of work items.
__global__ void k_cand_scan(const int* __restrict__ gcount, int ng, int* __restrict__ goff, int* __restrict__ cursor,
                            int* __restrict__ gblk)
{
    if (threadIdx.x != 0 || blockIdx.x != 0) return;
    int off = 0, blk = 0;
    for (int g = 0; g < ng; ++g) {
        goff[g] = off;
        cursor[g] = off;
        gblk[g] = blk;
        off += gcount[g];
        blk += (gcount[g] + kSubPerBlock - 1) / kSubPerBlock;
    }
    gblk[ng] = blk;
}

// Scatter into the group lists: ranks within the workgroup from LDS atomics,
// one global atomic per (workgroup, group) for the base.
__global__ __launch_bounds__(1024) void k_cand_scatter(const uint32_t* __restrict__ cand, int64_t n_sub, int ng,
                                                       int* __restrict__ cursor, int* __restrict__ pairs)
{
    __shared__ int h[kMaxGroups];
    __shared__ int base[kMaxGroups];
    if (threadIdx.x < kMaxGroups) h[threadIdx.x] = 0;
    __syncthreads();
    uint32_t w[kBucketItems];
    int rk[kBucketItems][3];
#pragma unroll
    for (int r = 0; r < kBucketItems; ++r) {
        const int64_t s = ((int64_t)blockIdx.x * kBucketItems + r) * 1024 + threadIdx.x;
        w[r] = s < n_sub ? cand[s] : 0u;
        const int n = (int)(w[r] & 3u);
#pragma unroll
        for (int j = 0; j < 3; ++j) rk[r][j] = j < n ? atomicAdd(&h[(w[r] >> (8 * (j + 1))) & 0xFFu], 1) : 0;
    }
    __syncthreads();
    if ((int)threadIdx.x < ng) base[threadIdx.x] = h[threadIdx.x] ? atomicAdd(&cursor[threadIdx.x], h[threadIdx.x]) : 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kBucketItems; ++r) {
        const int64_t s = ((int64_t)blockIdx.x * kBucketItems + r) * 1024 + threadIdx.x;
        const int n = (int)(w[r] & 3u);
#pragma unroll
        for (int j = 0; j < 3; ++j)
            if (j < n) pairs[base[(w[r] >> (8 * (j + 1))) & 0xFFu] + rk[r][j]] = (int)(s * 4 + j);
    }
}

// Search of the candidate groups in the general three-MFMA form: work item w
// (grid-stride over workgroups) is up to kSubPerBlock consecutive entries of
// one group's list; the workgroup stages the group's chunks of the split
// codebook in LDS and each wavefront searches 32 entries with per-slot
// tracking, as the short-codebook search does.  Per entry (s, j): the lane
// pair's best score, second best, best index and S_sc go to
// part[j * n_sub + s].
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_refine_h16(
    const float* __restrict__ X, const float* __restrict__ hcol, const uint8_t* __restrict__ mask, int64_t n_sub,
    int64_t nb, int d, const uint4* __restrict__ P, const float* __restrict__ cmax, int nchunks, int ng,
    const int* __restrict__ gcount, const int* __restrict__ goff, const int* __restrict__ gblk,
    const int* __restrict__ pairs, float4* __restrict__ part)
{
    constexpr int kChunkVec = kChunkTiles * 128;                 // uint4 per chunk
    __shared__ uint4 lds[kGroupChunks * kChunkVec];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int a_off = half * 32 + (lane & 31);
    const float cm = *cmax;
    const int T = gblk[ng];
    for (int w = blockIdx.x; w < T; w += gridDim.x) {
        int lo = 0, hi = ng;                                      // gblk[lo] <= w < gblk[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (gblk[mid] <= w) lo = mid; else hi = mid;
        }
        const int g = lo;
        const int first = (w - gblk[g]) * kSubPerBlock;
        const int cnt = min(kSubPerBlock, gcount[g] - first);
        const int c0 = g * kGroupChunks;
        const int ncg = min(kGroupChunks, nchunks - c0);
        __syncthreads();                                          // the previous item's tiles are read
        for (int i = threadIdx.x; i < ncg * kChunkVec; i += kWaves * 64) lds[i] = P[(size_t)c0 * kChunkVec + i];
        __syncthreads();
        if (wave * kSubPerWave >= cnt) continue;                  // wave-uniform
        const int qi = wave * kSubPerWave + (lane & 31);
        const bool valid = qi < cnt;
        const int e = valid ? pairs[goff[g] + first + qi] : 0;
        const int64_t s = e >> 2;
        const int j = e & 3;
        h16x8 bh, bl;
        float S_sc;
        int shift_s;
        general_operand(X, hcol, mask, s, nb, d, valid, half, cm, bh, bl, S_sc, shift_s);
        float b1 = __builtin_inff(), b2 = __builtin_inff();
        int kt1 = 0;
        float pk[16];
#pragma unroll
        for (int t = 0; t < 16; ++t) pk[t] = __builtin_inff();
        f32x16 accA, accB;
        for (int t = 0; t < 16; ++t) accB[t] = __builtin_inff();
        const int kt0 = c0 * kChunkTiles;
        int ktB = kt0;
        const uint4* L = lds + a_off;
#pragma unroll 1
        for (int tt = 0; tt < ncg * kChunkTiles; tt += 2) {
            const uint4* A0 = L + tt * 128;
            const uint4* A1 = A0 + 128;
            const h16x8 ah0 = __builtin_bit_cast(h16x8, A0[0]);
            const h16x8 al0 = __builtin_bit_cast(h16x8, A0[64]);
            accA = tile_h16<true>(ah0, al0, bh, bl, accB, ktB, b1, b2, kt1, pk);
            const h16x8 ah1 = __builtin_bit_cast(h16x8, A1[0]);
            const h16x8 al1 = __builtin_bit_cast(h16x8, A1[64]);
            accB = tile_h16<true>(ah1, al1, bh, bl, accA, kt0 + tt, b1, b2, kt1, pk);
            ktB = kt0 + tt + 1;
        }
        track<true>(accB, ktB, b1, b2, kt1, pk);
        park_resolve(pk, b1, b2, kt1);
        // merge of the lane pair (the two halves hold the tile's two row sets)
        const int jb = kt1 & 15;
        const int kb = (kt1 >> 4) * kTile + (jb >> 2) * 8 + half * 4 + (jb & 3);
        const float ob1 = __shfl_xor(b1, 32);
        const float ob2 = __shfl_xor(b2, 32);
        const int okb = __shfl_xor(kb, 32);
        float gb, gs;
        int gk;
        if (b1 < ob1 || (b1 == ob1 && kb < okb)) {
            gb = b1; gk = kb; gs = fminf(b2, ob1);
        } else {
            gb = ob1; gk = okb; gs = fminf(ob2, b1);
        }
        if (half == 0 && valid) part[(size_t)j * n_sub + s] = make_float4(gb, gs, __int_as_float(gk), S_sc);
    }
}

// Per sub-vector with candidates: the lexicographic (score, index) minimum
// over its candidates' results and the second best over the rest, certified
// with the search's bound; certified winners are written, the rest go to the
// exact re-search.  Outside the candidate groups every exact score lies
// above the exact minimum, so a winner certified among the candidates is the
// exact argmin over the whole codebook.
__global__ __launch_bounds__(256) void k_cand_merge(
    const float* __restrict__ X, const float* __restrict__ hcol, const float* __restrict__ rho,
    const uint8_t* __restrict__ mask, int64_t nb, int d, const float* __restrict__ C, int K, int64_t n_sub,
    const uint32_t* __restrict__ cand, const float4* __restrict__ part, uint16_t* __restrict__ idx,
    float* __restrict__ dist, int* __restrict__ flag_count, int* __restrict__ flag_list)
{
    const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int lane = threadIdx.x & 63;
    bool flag = false;
    if (s < n_sub) {
        const uint32_t w = cand[s];
        const int n = (int)(w & 3u);
        if (n) {
            const float4 p0 = part[s];
            float gb = p0.x, gs = p0.y;
            int gk = __float_as_int(p0.z);
            const float S_sc = p0.w;
            for (int j = 1; j < n; ++j) {
                const float4 q = part[(size_t)j * n_sub + s];
                const int qk = __float_as_int(q.z);
                if (q.x < gb || (q.x == gb && qk < gk)) {
                    gs = fminf(q.y, gb);
                    gb = q.x;
                    gk = qk;
                } else {
                    gs = fminf(gs, q.x);
                }
            }
            const float u = 5.9604644775390625e-8f;   // 2^-24
            const float eb = 48.f * u * (9.f * S_sc + 4.f * fmaxf(gb, -S_sc)) + 1.f;
            const float es = 48.f * u * (9.f * S_sc + 4.f * fmaxf(gs, -S_sc)) + 1.f;
            if ((gs - gb) > (eb + es) && gk < K) {
                idx[s] = (uint16_t)gk;
                if (dist) {
                    double omd[8];
                    float xs[8];
                    exact_weights(hcol, rho, mask, s, nb, d, omd);
                    for (int t = 0; t < d; ++t) xs[t] = X[s * d + t];
                    dist[s] = (float)exact_dist(omd, xs, C + (size_t)gk * d, d);
                }
            } else {
                flag = true;
            }
        }
    }
    list_append(flag, lane, s, flag_count, flag_list);
}

// Chunk minima of the flagged sub-vectors (long codebooks).  The general
// three-MFMA form of the search over the flag list, entries [0, min(count,
// cap)): workgroup = the next kSubPerBlock entries (grid-stride over x) times
// kCminChunks consecutive chunks of the split codebook (y), staged through
// LDS one chunk at a time with the next one loaded into registers.  Per
// (entry, chunk): the smallest scaled score over the chunk's centroids (both
// halves of the lane pair); per entry its S_sc, the scale of the rounding
// bound err(e) = 48u (9 S_sc + 4 max(e, -S_sc)) + 1 that the search's
// certification uses.
__global__ __launch_bounds__(kWaves * 64) void k_assign_cmin(
    const float* __restrict__ X, const float* __restrict__ hcol, const uint8_t* __restrict__ mask, int64_t nb, int d,
    const uint4* __restrict__ P, const float* __restrict__ cmax, int nchunks, const int* __restrict__ list,
    const int* __restrict__ list_count, int cap, float* __restrict__ cmin, float* __restrict__ ssc)
{
    constexpr int kChunkVec = kChunkTiles * 128;                 // uint4 per chunk
    __shared__ uint4 lds[2][kChunkVec];
    const int64_t count = min(*list_count, cap);
    const int c0 = blockIdx.y * kCminChunks;
    const int c1 = min(nchunks, c0 + kCminChunks);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int a_off = half * 32 + (lane & 31);
    for (int64_t lb = blockIdx.x; lb * kSubPerBlock < count; lb += gridDim.x) {
        const int64_t q = lb * kSubPerBlock + wave * kSubPerWave + (lane & 31);
        const bool valid = q < count;
        const int64_t s = valid ? (int64_t)list[q] : 0;
        h16x8 bh, bl;
        float S_sc;
        int shift_s;
        general_operand(X, hcol, mask, s, nb, d, valid, half, *cmax, bh, bl, S_sc, shift_s);
        if (blockIdx.y == 0 && half == 0 && valid) ssc[q] = S_sc;
        __syncthreads();                                          // the previous entries' last chunk is read
        uint4 pre0 = P[(size_t)c0 * kChunkVec + threadIdx.x];
        uint4 pre1 = P[(size_t)c0 * kChunkVec + threadIdx.x + kWaves * 64];
        lds[0][threadIdx.x] = pre0;
        lds[0][threadIdx.x + kWaves * 64] = pre1;
        __syncthreads();
        for (int c = c0; c < c1; ++c) {
            if (c + 1 < c1) {
                const uint4* src = P + (size_t)(c + 1) * kChunkVec;
                pre0 = src[threadIdx.x];
                pre1 = src[threadIdx.x + kWaves * 64];
            }
            const uint4* L = lds[(c - c0) & 1] + a_off;
            float cm = __builtin_inff();
#pragma unroll 2
            for (int tt = 0; tt < kChunkTiles; ++tt) {
                const uint4* A0 = L + tt * 128;
                const h16x8 ah = __builtin_bit_cast(h16x8, A0[0]);
                const h16x8 al = __builtin_bit_cast(h16x8, A0[64]);
                f32x16 acc = {};
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bl, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, acc, 0, 0, 0);
                cm = fminf(cm, tile_min(acc));
            }
            cm = fminf(cm, __shfl_xor(cm, 32));
            if (half == 0 && valid) cmin[(size_t)q * nchunks + c] = cm;
            if (c + 1 < c1) {
                lds[(c + 1 - c0) & 1][threadIdx.x] = pre0;
                lds[(c + 1 - c0) & 1][threadIdx.x + kWaves * 64] = pre1;
            }
            __syncthreads();
        }
    }
}

// Exact search of the flagged sub-vectors over their candidate chunks: one
// wavefront per entry of [0, min(count, cap)) (grid-stride).  With gm the
// smallest chunk minimum, chunk c is a candidate unless (cm_c - gm) >
// err(cm_c) + err(gm), the search's certification applied to chunk minima:
// every centroid of a non-candidate chunk has an exact score above the
// sub-vector's exact minimum (a - err(a) grows with a), so no minimizer and
// no tie is left out.  Every centroid of the candidate chunks is evaluated
// in float64 in the direct form (terms in t order, exactly as a plain
// float64 evaluation rounds) and the lexicographic (D, k) minimum is the
// exact argmin with ties to the lowest index.
__global__ __launch_bounds__(256) void k_exact_chunks(
    const float* __restrict__ X, const float* __restrict__ hcol, const float* __restrict__ rho,
    const uint8_t* __restrict__ mask, int64_t nb, int d, const float* __restrict__ C, int K, int nchunks,
    const int* __restrict__ list, const int* __restrict__ list_count, int cap, const float* __restrict__ cmin,
    const float* __restrict__ ssc, uint16_t* __restrict__ idx, float* __restrict__ dist)
{
    const int64_t count = min(*list_count, cap);
    const int lane = threadIdx.x & 63;
    const int64_t waves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const float u = 5.9604644775390625e-8f;   // 2^-24
    const bool vecC = d == 8 && (reinterpret_cast<uintptr_t>(C) & 15u) == 0;
    for (int64_t q = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); q < count; q += waves) {
        const int64_t s = list[q];
        const float S = ssc[q];
        const float* cm = cmin + (size_t)q * nchunks;
        float gm = __builtin_inff();
        for (int c = lane; c < nchunks; c += 64) gm = fminf(gm, cm[c]);
        for (int off = 32; off > 0; off >>= 1) gm = fminf(gm, __shfl_xor(gm, off));
        const float eg = 48.f * u * (9.f * S + 4.f * fmaxf(gm, -S)) + 1.f;
        double om[8];
        float x[8];
        exact_weights(hcol, rho, mask, s, nb, d, om);
        for (int t = 0; t < d; ++t) x[t] = X[s * d + t];
        double bd = __builtin_inf();
        int bk = K;
        for (int cb = 0; cb < nchunks; cb += 64) {
            bool cand = false;
            if (cb + lane < nchunks) {
                const float v = cm[cb + lane];
                const float ev = 48.f * u * (9.f * S + 4.f * fmaxf(v, -S)) + 1.f;
                cand = !((v - gm) > (ev + eg));               // NaN keeps the chunk
            }
            unsigned long long ball = __ballot(cand);
            while (ball) {
                const int c = cb + __ffsll((long long)ball) - 1;
                ball &= ball - 1ull;
                const int kbeg = c * kChunkTiles * kTile;
                const int kend = min(K, kbeg + kChunkTiles * kTile);
                constexpr int kPerLane = kChunkTiles * kTile / 64;   // 4 centroids of the chunk per lane
                if (vecC) {
                    // the lane's rows are all requested before any is used
                    float cr[kPerLane][8];
#pragma unroll
                    for (int j = 0; j < kPerLane; ++j) {
                        const int k = kbeg + lane + 64 * j;
                        const int kk = k < kend ? k : kbeg;
                        const float4 ca = reinterpret_cast<const float4*>(C)[(size_t)kk * 2];
                        const float4 cb4 = reinterpret_cast<const float4*>(C)[(size_t)kk * 2 + 1];
                        cr[j][0] = ca.x; cr[j][1] = ca.y; cr[j][2] = ca.z; cr[j][3] = ca.w;
                        cr[j][4] = cb4.x; cr[j][5] = cb4.y; cr[j][6] = cb4.z; cr[j][7] = cb4.w;
                    }
#pragma unroll
                    for (int j = 0; j < kPerLane; ++j) {
                        const int k = kbeg + lane + 64 * j;
                        if (k >= kend) continue;
                        const double D = exact_dist(om, x, cr[j], d);
                        if (D < bd || (D == bd && k < bk)) { bd = D; bk = k; }
                    }
                } else {
                    for (int k = kbeg + lane; k < kend; k += 64) {
                        const double D = exact_dist(om, x, C + (size_t)k * d, d);
                        if (D < bd || (D == bd && k < bk)) { bd = D; bk = k; }
                    }
                }
            }
        }
        for (int off = 32; off > 0; off >>= 1) {
            const double od = __shfl_xor(bd, off);
            const int ok = __shfl_xor(bk, off);
            if (od < bd || (od == bd && ok < bk)) { bd = od; bk = ok; }
        }
        if (lane == 0) {
            idx[s] = (uint16_t)bk;
            if (dist) dist[s] = (float)bd;
        }
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
    uint16_t* __restrict__ idx, float* __restrict__ dist, int vecC, int start)
{
    const int n = *flag_count;
    const int lane = threadIdx.x & 63;
    const float u = 5.9604644775390625e-8f;
    const int waves = gridDim.x * (blockDim.x >> 6);
    for (int f = start + blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); f < n; f += waves) {
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
// Workgroups of the one-chunk search (16 per CU on 256 CUs; 2048-8192 measured alike).
constexpr unsigned kOneBlocks = 4096;
// Row sets of 32 per wave in the shared-weight search, and rows per workgroup.
constexpr int kSharedSets = 4;
constexpr int kSharedRows = kSubPerBlock * kSharedSets;
// Row sets of 32 per wave in the coarse pass (no accumulator ping-pong, so
// twice the sets fit, and the chunk staging serves twice the rows).
constexpr int kCoarseSets = 8;
constexpr int kCoarseRows = kSubPerBlock * kCoarseSets;

inline int padded_K(int K) { return (K + kChunkK - 1) / kChunkK * kChunkK; }

// Arrays of the two-pass search, taken from the workspace beyond
// ws_assign's size when there is room: cand (4 bytes per sub-vector), the
// group lists (up to three entries per sub-vector), the candidates' results
// (three float4 per sub-vector) and the per-group counters.
size_t ws_coarse(int64_t n_sub)
{
    return align_up((size_t)n_sub * 4) + align_up((size_t)n_sub * 3 * 4) + align_up((size_t)n_sub * 3 * 16) +
           4 * align_up(sizeof(int) * (kMaxGroups + 1));
}

// Workspace an assignment uses at most: ws_assign plus the two-pass search's
// arrays and the chunk path's room for flagged sub-vectors.
size_t ws_assign_full(int64_t n_sub, int K)
{
    const int nch = padded_K(K) / kChunkK;
    return ws_assign(n_sub, K) + ws_coarse(n_sub) +
           align_up((size_t)kCminCap * ((size_t)nch + 1) * sizeof(float)) + 4 * kAlign;
}

size_t ws_assign(int64_t n_sub, int K)
{
    // split codebook (64 bytes per centroid), flag counter, flag list, max |c|,
    // partial maxima, dirty counter, dirty list, block pattern words (4 bytes
    // per column block: at most n_sub bytes when there are 4 rows or more;
    // fewer rows do not classify blocks)
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
    // blocks are classified when there are at least 4 rows (their pattern
    // words then fit in the n_sub bytes the workspace holds for them)
    const bool classify = mask != nullptr && M >= 4;
    uint32_t* pattern = classify ? cv.take<uint32_t>((size_t)nb) : nullptr;
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
        if (!slot && mask && !classify) {
            // long codebook, masked, fewer than 4 rows: the general form for all
            hipLaunchKernelGGL(k_assign_h16<false>, dim3(grid_for(n_sub, kSubPerBlock)), dim3(kWaves * 64), 0, st, X,
                               hcol, rho, mask, n_sub, nb, d, P, cmax, C, K, nch, nullptr, nullptr, idx, dist,
                               flag_count, flag_list);
            VQ_LAUNCHED("k_assign_h16");
        } else if (slot) {
            // short codebooks: one pass of the general form (the block
            // classification would cost more than the shared form saves)
            if (nch == 1) {
                // one chunk: staged once per workgroup, groups taken in turn
                const unsigned groups = grid_for(n_sub, kSubPerBlock);
                hipLaunchKernelGGL(k_assign_h16_one, dim3(std::min(groups, kOneBlocks)), dim3(kWaves * 64), 0, st, X,
                                   hcol, rho, mask, n_sub, nb, d, P, cmax, C, K, idx, dist, flag_count, flag_list);
                VQ_LAUNCHED("k_assign_h16_one");
            } else {
                hipLaunchKernelGGL(k_assign_h16<true>, dim3(grid_for(n_sub, kSubPerBlock)), dim3(kWaves * 64), 0, st,
                                   X, hcol, rho, mask, n_sub, nb, d, P, cmax, C, K, nch, nullptr, nullptr, idx, dist,
                                   flag_count, flag_list);
                VQ_LAUNCHED("k_assign_h16");
            }
        } else {
        if (mask) {
            hipLaunchKernelGGL(k_block_pattern, dim3((unsigned)nb), dim3(256), 0, st, mask, M, nb, pattern);
            VQ_LAUNCHED("k_block_pattern");
            hipLaunchKernelGGL(k_dirty, dim3(grid_for(n_sub, 4096)), dim3(1024), 0, st, mask, pattern, n_sub,
                               (uint32_t)nb, dirty_count, dirty_list);
            VQ_LAUNCHED("k_dirty");
        }
        // Two passes when the workspace has room for them: the coarse pass
        // (one MFMA per tile) names each sub-vector's candidate groups, the
        // groups are searched in the general form over their lists only,
        // and the merge certifies the winners.
        const int ng = (nch + kGroupChunks - 1) / kGroupChunks;
        const size_t room = cv.cap > cv.used + 8 * kAlign ? cv.cap - cv.used - 8 * kAlign : 0;
        const bool two_pass = ng <= kMaxGroups && n_sub < ((int64_t)1 << 29) && room >= ws_coarse(n_sub);
        if (two_pass) {
            uint32_t* cand = cv.take<uint32_t>((size_t)n_sub);
            int* pairs = cv.take<int>((size_t)n_sub * 3);
            float4* partv = cv.take<float4>((size_t)n_sub * 3);
            int* gcount = cv.take<int>(kMaxGroups + 1);
            int* goff = cv.take<int>(kMaxGroups + 1);
            int* cursor = cv.take<int>(kMaxGroups + 1);
            int* gblk = cv.take<int>(kMaxGroups + 1);
            if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_assign: workspace too small");
            hipLaunchKernelGGL(k_fill_int, dim3(1), dim3(kMaxGroups + 1), 0, st, gcount, kMaxGroups + 1, 0);
            VQ_LAUNCHED("k_fill_int");
            const int64_t coarse_groups = (M + kCoarseRows - 1) / kCoarseRows * nb;
            hipLaunchKernelGGL((k_assign_h16s<false, kCoarseSets, true>), dim3((unsigned)coarse_groups),
                               dim3(kWaves * 64), 0, st, X, hcol, rho, mask, mask ? pattern : nullptr, M, nb, d, P,
                               cmax, C, K, nch, idx, dist, flag_count, flag_list, dirty_count, dirty_list, cand);
            VQ_LAUNCHED("k_assign_h16s");
            const unsigned gb = grid_for(n_sub, 1024 * kBucketItems);
            hipLaunchKernelGGL(k_cand_count, dim3(gb), dim3(1024), 0, st, cand, n_sub, ng, gcount);
            VQ_LAUNCHED("k_cand_count");
            hipLaunchKernelGGL(k_cand_scan, dim3(1), dim3(64), 0, st, gcount, ng, goff, cursor, gblk);
            VQ_LAUNCHED("k_cand_scan");
            hipLaunchKernelGGL(k_cand_scatter, dim3(gb), dim3(1024), 0, st, cand, n_sub, ng, cursor, pairs);
            VQ_LAUNCHED("k_cand_scatter");
            hipLaunchKernelGGL(k_refine_h16, dim3(kRefineBlocks), dim3(kWaves * 64), 0, st, X, hcol, mask, n_sub, nb,
                               d, P, cmax, nch, ng, gcount, goff, gblk, pairs, partv);
            VQ_LAUNCHED("k_refine_h16");
            hipLaunchKernelGGL(k_cand_merge, dim3(grid_for(n_sub, 256)), dim3(256), 0, st, X, hcol, rho, mask, nb, d,
                               C, K, n_sub, cand, partv, idx, dist, flag_count, flag_list);
            VQ_LAUNCHED("k_cand_merge");
        } else {
            // sub-vectors with their block's weights: two MFMAs per tile
            hipLaunchKernelGGL((k_assign_h16s<false, kSharedSets, false>), dim3((unsigned)shared_groups),
                               dim3(kWaves * 64), 0, st, X, hcol, rho, mask, mask ? pattern : nullptr, M, nb, d, P,
                               cmax, C, K, nch, idx, dist, flag_count, flag_list, nullptr, nullptr, nullptr);
            VQ_LAUNCHED("k_assign_h16s");
        }
        // the rest, each with its own weights (and, after the coarse pass, the
        // sub-vectors with more than three candidate groups): three MFMAs per tile
        if (mask || two_pass) {
            hipLaunchKernelGGL(k_assign_h16<false>, dim3(grid_for(n_sub, kSubPerBlock)), dim3(kWaves * 64), 0, st, X,
                               hcol, rho, mask, n_sub, nb, d, P, cmax, C, K, nch, dirty_list, dirty_count, idx, dist,
                               flag_count, flag_list);
            VQ_LAUNCHED("k_assign_h16");
        }
        }
    }
    // Long codebooks: the first flagged sub-vectors (as many as the workspace
    // holds beyond its required size, at most kCminCap) take the chunk path:
    // chunk minima on the matrix cores, then float64 over the candidate
    // chunks only.  The rest (or all, without room) scan the whole codebook.
    const int nch = Kpad / kChunkK;
    int cap = 0;
    if (nch > kSlotChunks) {
        const size_t per = (size_t)nch * sizeof(float) + sizeof(float);
        const size_t room = cv.cap > cv.used + 4 * kAlign ? cv.cap - cv.used - 4 * kAlign : 0;
        cap = (int)std::min<size_t>((size_t)kCminCap, std::min<size_t>(room / per, (size_t)n_sub));
        if (cap < kSubPerBlock) cap = 0;
    }
    if (cap > 0) {
        float* cmin = cv.take<float>((size_t)cap * nch);
        float* ssc = cv.take<float>((size_t)cap);
        if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_assign: workspace too small");
        const dim3 gc((unsigned)std::min<int64_t>(kCminListBlocks, (cap + kSubPerBlock - 1) / kSubPerBlock),
                      (unsigned)((nch + kCminChunks - 1) / kCminChunks));
        hipLaunchKernelGGL(k_assign_cmin, gc, dim3(kWaves * 64), 0, st, X, hcol, mask, nb, d, P, cmax, nch, flag_list,
                           flag_count, cap, cmin, ssc);
        VQ_LAUNCHED("k_assign_cmin");
        hipLaunchKernelGGL(k_exact_chunks, dim3((unsigned)std::min<int64_t>((cap + 3) / 4, kExactBlocks)), dim3(256),
                           0, st, X, hcol, rho, mask, nb, d, C, K, nch, flag_list, flag_count, cap, cmin, ssc, idx,
                           dist);
        VQ_LAUNCHED("k_exact_chunks");
    }
    const unsigned gx = (unsigned)std::min<int64_t>((n_sub + 3) / 4, kExactBlocks);
    const int vecC = (d == 8 && (reinterpret_cast<uintptr_t>(C) & 15u) == 0) ? 1 : 0;
    hipLaunchKernelGGL(k_assign_exact, dim3(gx), dim3(256), 0, st, X, hcol, rho, mask, nb, d, C, K,
                       flag_count, flag_list, idx, dist, vecC, cap);
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

// Ids of the sub-vectors the last search sent to the exact path: the count,
// and up to cap of the ids copied to the host (diagnostics).
vq_status assign_flag_list(void* ws, size_t ws_bytes, int64_t n_sub, int K, int32_t* out, int64_t cap,
                           int64_t* count, hipStream_t st)
{
    Carver cv(ws, ws_bytes);
    cv.take<uint4>((size_t)padded_K(K) * 4);
    int* flag_count = cv.take<int>(1);
    int* flag_list = cv.take<int>((size_t)n_sub);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "workspace too small");
    int n = 0;
    VQ_HIP(hipMemcpyAsync(&n, flag_count, sizeof(int), hipMemcpyDeviceToHost, st));
    VQ_HIP(hipStreamSynchronize(st));
    if (n < 0 || (int64_t)n > n_sub) return fail(VQ_ERR_INVALID, "no assignment recorded in this workspace");
    const int64_t m = std::min<int64_t>(n, cap);
    if (m > 0) {
        VQ_HIP(hipMemcpyAsync(out, flag_list, sizeof(int32_t) * (size_t)m, hipMemcpyDeviceToHost, st));
        VQ_HIP(hipStreamSynchronize(st));
    }
    *count = n;
    return VQ_OK;
}


// ---- allocation-free assignment ---------------------------------------------
// For callers that cannot allocate device memory (code under stream capture,
// tight serving loops): the workspace of an assignment lives in one
// file-scope device array per GPU, held until the process ends.  Host code
// never passes the array's name to a kernel (on the host it only stands in for
// the symbol); it fetches the array's device address once per device, with
// that device current, and uses that address everywhere.  The kernels clear
// the counters they use at the start of every call; calls that overlap on one
// GPU share the array and race.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // per device: the array's device address
}  // namespace

size_t assign_scratch_bytes() { return kScratchBytes; }

vq_status scratch_address(void** out)
{
    int dev = -1;
    VQ_HIP(hipGetDevice(&dev));
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (p == nullptr) return fail(VQ_ERR_DEVICE, "hipGetSymbolAddress(scratch) returned a null address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return VQ_OK;
}

// vq_assign with the file-scope array as its workspace; sizes already checked
// against kScratchBytes by the caller.
vq_status assign_noalloc_launch(const float* X, const float* hcol, const float* rho, const uint8_t* mask,
                                int64_t M, int64_t N, int d, const float* C, int K, uint16_t* idx, float* dist,
                                hipStream_t st)
{
    void* ws = nullptr;
    if (vq_status s = scratch_address(&ws); s != VQ_OK) return s;
    return assign_launch(X, hcol, rho, mask, M, N, d, C, K, idx, dist, ws, kScratchBytes, st);
}

}  // namespace vq
