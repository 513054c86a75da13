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

constexpr int kWaves = 8;                 // waves per workgroup
constexpr int kSubPerWave = 32;           // sub-vectors per wave (MFMA B columns)
constexpr int kSubPerBlock = kWaves * kSubPerWave;
constexpr int kTile = 32;                 // centroids per MFMA tile (A rows)
constexpr int kChunkTiles = 8;            // tiles staged in LDS at once
constexpr float kPadSq = 1.0e30f;         // c*c of padding centroids
constexpr int kExactBlocks = 2048;

// P[k] = 16 floats in two halves, one per half-wavefront of the MFMA A
// operand: [-2c_0, -2c_2, -2c_4, -2c_6, c_0^2, c_2^2, c_4^2, c_6^2] then the
// same for the odd dimensions.  Dimensions >= d are 0; padding centroids
// (k >= K) have -2c = 0 and c^2 = kPadSq.  Also clears the flag counter.
__global__ void k_cb_prep(const float* __restrict__ C, int K, int d, int Kpad,
                          float* __restrict__ P, int* __restrict__ flag_count, int* __restrict__ dirty_count)
{
    int k = blockIdx.x * blockDim.x + threadIdx.x;
    if (k == 0) {
        *flag_count = 0;
        *dirty_count = 0;
    }
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
        const int h = t & 1, q = t >> 1;
        p[h * 8 + q] = m2c;
        p[h * 8 + 4 + q] = sq;
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

// Minimum of a tile's 16 accumulator values (min3 chains).
__device__ __forceinline__ float tile_min(const f32x16& a)
{
    float m0 = fminf(fminf(a[0], a[1]), a[2]);
    float m1 = fminf(fminf(a[3], a[4]), a[5]);
    float m2 = fminf(fminf(a[6], a[7]), a[8]);
    float m3 = fminf(fminf(a[9], a[10]), a[11]);
    float m4 = fminf(fminf(a[12], a[13]), a[14]);
    m0 = fminf(fminf(m0, m1), m2);
    m3 = fminf(fminf(m3, m4), a[15]);
    return fminf(m0, m3);
}

// Exact update of this lane's (best, second best, best position) with the
// 16 values of tile kt, in slot order (slot order is centroid order within
// the lane, so equal values keep the lower index).  Position = kt*16 + slot.
__device__ __forceinline__ void lane_update(const f32x16& a, int kt, float& b1, float& b2, int& kbp)
{
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float v = a[j];
        const bool lt = v < b1;
        b2 = __builtin_amdgcn_fmed3f(b1, b2, v);
        b1 = lt ? v : b1;
        kbp = lt ? kt * 16 + j : kbp;
    }
}

// One 32x32 tile in the general form: eight chained MFMAs over the 16 terms
// (4 pairs of -2c_t * omega_t x_t, then 4 pairs of c_t^2 * omega_t).  The
// previous tile's minimum is formed between the MFMAs; only if it beats the
// lane's second best (rare once the search has seen a few tiles) does the
// wave walk that tile's values.
// a0 = this lane's 4 values of -2c, a1 = its 4 values of c^2; bw = omega*x,
// bo = omega for this lane's 4 dimensions.
__device__ __forceinline__ f32x16 tile_general(const float4 a0, const float4 a1, const float* bw, const float* bo,
                                               const f32x16& prev, int ktp, float& b1, float& b2, int& kbp)
{
    f32x16 acc = {};
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.x, bw[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.y, bw[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.z, bw[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.w, bw[3], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a1.x, bo[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a1.y, bo[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a1.z, bo[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a1.w, bo[3], acc, 0, 0, 0);
    const float tm = tile_min(prev);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);   // one VALU
    }
    if (tm < b2) lane_update(prev, ktp, b1, b2, kbp);
    return acc;
}

// The same tile when every sub-vector of the wavefront has the same weights
// omega (same column block, same mask byte): the centroid term
// sum_t omega_t c_t^2 is a per-centroid bias, formed here with 4 FMAs per
// lane (each half-wave sums its 4 dimensions) and added by a fifth MFMA
// against a B row of ones, so the tile needs 5 MFMAs instead of 8.
__device__ __forceinline__ f32x16 tile_shared(const float4 a0, const float4 a1, const float* bw, const float* wo,
                                              const f32x16& prev, int ktp, float& b1, float& b2, int& kbp)
{
    float bias = a1.x * wo[0];
    bias = fmaf(a1.y, wo[1], bias);
    bias = fmaf(a1.z, wo[2], bias);
    bias = fmaf(a1.w, wo[3], bias);
    f32x16 acc = {};
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.x, bw[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.y, bw[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.z, bw[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a0.w, bw[3], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(bias, 1.0f, acc, 0, 0, 0);
    const float tm = tile_min(prev);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);   // two VALU
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (tm < b2) lane_update(prev, ktp, b1, b2, kbp);
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

// Workgroup = kWaves wavefronts x 32 sub-vectors, searched against the
// whole codebook.
//   SHARED: wavefront w takes wave group g = blockIdx.x * kWaves + w, i.e.
//     32 consecutive rows of column block b; all lanes use the block's
//     majority weight pattern (5-MFMA tile).  A lane whose own mask byte
//     differs is computed but not written: it is in the list of the
//     general kernel.
//   general: lane l of wavefront w takes sub-vector list[(blockIdx.x *
//     kWaves + w) * 32 + (l & 31)] with its own weights (8-MFMA tile).
// The expanded codebook (padded to whole chunks) streams through LDS in
// chunks of kChunkTiles*32 centroids, double buffered: the next chunk is
// fetched into registers while the current one is searched, so there is one
// barrier per chunk.  Within a wave the tiles are software pipelined: tile
// t's MFMAs are issued with tile t-1's argmin updates between them (two
// accumulators alternate).
template <bool SHARED>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_assign_mfma(
    const float* __restrict__ X, const float* __restrict__ hcol, const float* __restrict__ rho,
    const uint8_t* __restrict__ mask, const uint8_t* __restrict__ pattern, int64_t M, int64_t nb, int d,
    const float4* __restrict__ P, const float* __restrict__ C, int K, int nchunks,
    const int* __restrict__ list, const int* __restrict__ list_count, int64_t groups,
    uint16_t* __restrict__ idx, float* __restrict__ dist,
    int* __restrict__ flag_count, int* __restrict__ flag_list)
{
    constexpr int kChunkVec = kChunkTiles * kTile * 4;          // float4 per chunk
    constexpr int kVecPerThread = kChunkVec / (kWaves * 64);
    static_assert(kChunkTiles % 2 == 0, "tiles are processed in pairs");
    static_assert(kVecPerThread == 2, "two float4 per thread per chunk");
    __shared__ float4 lds[2][kChunkVec];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int64_t e = (int64_t)blockIdx.x * kWaves + wave;
    int64_t s = 0, b = 0;
    bool active, valid;
    unsigned mb = 0u, pat = 0u;
    if (SHARED) {
        if ((int64_t)blockIdx.x * kWaves >= groups) return;      // whole workgroup idle
        active = e < groups;                                       // wave-uniform
        const int64_t g = active ? e : 0;
        const int64_t rg = g / nb;
        b = g - rg * nb;
        const int64_t i = rg * kSubPerWave + (lane & 31);
        valid = active && i < M;
        s = i * nb + b;
        pat = (active && pattern) ? pattern[b] : 0u;
        mb = (valid && mask) ? mask[s] : 0u;
    } else {
        const int64_t count = *list_count;
        if ((int64_t)blockIdx.x * kWaves * kSubPerWave >= count) return;
        const int64_t q = e * kSubPerWave + (lane & 31);
        active = e * kSubPerWave < count;                          // wave-uniform
        valid = q < count;
        s = valid ? (int64_t)list[q] : 0;
        b = s % nb;
        mb = (valid && mask) ? mask[s] : 0u;
    }
    // lanes that write their result (in SHARED, only those of the pattern)
    const bool owner = valid && (!SHARED || mb == pat);

    // ---- the sub-vector's weights, B operand and weighted energy S -----
    const unsigned wmask = SHARED ? pat : mb;
    float x[8], om[8];
    float S = 0.f;
    for (int t = 0; t < 8; ++t) {
        float xv = 0.f, w = 0.f;
        if (valid && t < d) {
            xv = X[s * d + t];
            w = ((wmask >> t) & 1u) ? 0.f : hcol[b * d + t];
        }
        x[t] = xv;
        om[t] = w;
        S += w * xv * xv;
    }
    // this lane's half of the inner dimension: dimensions t = 2q + half;
    // wo = the group's common weights (same for every lane in SHARED)
    float bw[4], bo[4], wo[4];
    for (int q = 0; q < 4; ++q) {
        const int t = 2 * q + half;
        bw[q] = om[t] * x[t];
        bo[q] = om[t];
        wo[q] = (SHARED && active && t < d && !((pat >> t) & 1u)) ? hcol[b * d + t] : 0.f;
    }

    float b1 = __builtin_inff(), b2 = __builtin_inff();
    int kbp = 0;

    float4 pre0 = P[threadIdx.x];
    float4 pre1 = P[threadIdx.x + kWaves * 64];
    lds[0][threadIdx.x] = pre0;
    lds[0][threadIdx.x + kWaves * 64] = pre1;
    __syncthreads();

    // accB holds the pending tile; +inf values leave the slots unchanged
    f32x16 accA, accB;
    for (int j = 0; j < 16; ++j) accB[j] = __builtin_inff();
    int ktB = 0;
    const int a_off = (lane & 31) * 4 + half * 2;
    for (int c = 0; c < nchunks; ++c) {
        if (c + 1 < nchunks) {
            const float4* src = P + (size_t)(c + 1) * kChunkVec;
            pre0 = src[threadIdx.x];
            pre1 = src[threadIdx.x + kWaves * 64];
        }
        if (active) {
            const float4* L = lds[c & 1] + a_off;
            const int kt0 = c * kChunkTiles;
#pragma unroll 1
            for (int tt = 0; tt < kChunkTiles; tt += 2) {
                const float4* A0 = L + tt * kTile * 4;
                const float4* A1 = A0 + kTile * 4;
                if (SHARED) {
                    accA = tile_shared(A0[0], A0[1], bw, wo, accB, ktB, b1, b2, kbp);
                    accB = tile_shared(A1[0], A1[1], bw, wo, accA, kt0 + tt, b1, b2, kbp);
                } else {
                    accA = tile_general(A0[0], A0[1], bw, bo, accB, ktB, b1, b2, kbp);
                    accB = tile_general(A1[0], A1[1], bw, bo, accA, kt0 + tt, b1, b2, kbp);
                }
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
    if (tile_min(accB) < b2) lane_update(accB, ktB, b1, b2, kbp);

    // ---- epilogue: best and second best of this sub-vector -------------
    // position kbp = tile * 16 + slot; slot j of this lane holds centroid row
    // (j/4)*8 + half*4 + j%4 of the tile
    const float sec = b2;
    const int jb = kbp & 15;
    const int kb = (kbp >> 4) * kTile + (jb >> 2) * 8 + half * 4 + (jb & 3);

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

    const bool writer = owner && half == 0;
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
        float x[8], om[8], bw[8];
        double w64[8];
        float S = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const bool on = t < d;
            x[t] = on ? X[s * d + t] : 0.f;
            om[t] = (on && !((mb >> t) & 1u)) ? hcol[b * d + t] : 0.f;
            bw[t] = om[t] * x[t];
            S += om[t] * x[t] * x[t];
            double w = (double)om[t];
            if (rho) w = w * rr;
            w64[t] = w;
        }
        float thr = __builtin_inff();
        double dbest = __builtin_inf();
        int arg = K;
        for (int k = lane; k < K; k += 64) {
            float c[8];
            if (vecC) {   // d == 8 and a 16-byte aligned codebook
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
            const float err = 32.f * u * (9.f * S + 4.f * fmaxf(e, -S)) + 1.0e-35f;
            if (e - err <= thr) {
                thr = fminf(thr, e + err);
                double acc = 0.0;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const double diff = (double)x[t] - (double)c[t];
                    const double sq = diff * diff;
                    acc = acc + w64[t] * sq;
                }
                if (acc < dbest) { dbest = acc; arg = k; }
            }
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

// Centroids per LDS chunk; the expanded codebook is padded to whole chunks.
constexpr int kChunkK = kChunkTiles * kTile;

inline int padded_K(int K) { return (K + kChunkK - 1) / kChunkK * kChunkK; }

size_t ws_assign(int64_t n_sub, int K)
{
    // expanded codebook, flag counter, flag list, dirty counter, dirty list,
    // block patterns (at most n_sub column blocks)
    return align_up((size_t)padded_K(K) * 16 * sizeof(float)) + align_up(sizeof(int)) +
           align_up((size_t)n_sub * sizeof(int)) + align_up(sizeof(int)) + align_up((size_t)n_sub * sizeof(int)) +
           align_up((size_t)n_sub);
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
    float* P = cv.take<float>((size_t)Kpad * 16);
    int* flag_count = cv.take<int>(1);
    int* flag_list = cv.take<int>((size_t)n_sub);
    int* dirty_count = cv.take<int>(1);
    int* dirty_list = cv.take<int>((size_t)n_sub);
    uint8_t* pattern = cv.take<uint8_t>((size_t)nb);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_assign: workspace too small");

    TimedRegion tr_all("assign", K, st);
    hipLaunchKernelGGL(k_cb_prep, dim3(grid_for(Kpad, 256)), dim3(256), 0, st, C, K, d, Kpad, P,
                       flag_count, dirty_count);
    VQ_LAUNCHED("k_cb_prep");
    {
        TimedRegion tr("assign_search", K, st);
        const int64_t groups = (M + kSubPerWave - 1) / kSubPerWave * nb;
        const float4* P4 = reinterpret_cast<const float4*>(P);
        const int nch = Kpad / kChunkK;
        if (mask) {
            hipLaunchKernelGGL(k_block_pattern, dim3((unsigned)nb), dim3(256), 0, st, mask, M, nb, pattern);
            VQ_LAUNCHED("k_block_pattern");
            hipLaunchKernelGGL(k_dirty, dim3(grid_for(n_sub, 4096)), dim3(1024), 0, st, mask, pattern, n_sub,
                               (uint32_t)nb, dirty_count, dirty_list);
            VQ_LAUNCHED("k_dirty");
        }
        hipLaunchKernelGGL(k_assign_mfma<true>, dim3(grid_for(groups, kWaves)), dim3(kWaves * 64), 0, st, X, hcol,
                           rho, mask, mask ? pattern : nullptr, M, nb, d, P4, C, K, nch, nullptr, nullptr, groups,
                           idx, dist, flag_count, flag_list);
        VQ_LAUNCHED("k_assign_mfma<shared>");
        if (mask) {
            hipLaunchKernelGGL(k_assign_mfma<false>, dim3(grid_for(n_sub, kSubPerBlock)), dim3(kWaves * 64), 0, st,
                               X, hcol, rho, mask, nullptr, M, nb, d, P4, C, K, nch, dirty_list, dirty_count, groups,
                               idx, dist, flag_count, flag_list);
            VQ_LAUNCHED("k_assign_mfma<general>");
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
    cv.take<float>((size_t)padded_K(K) * 16);
    int* flag_count = cv.take<int>(1);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "workspace too small");
    VQ_HIP(hipMemcpyAsync(out, flag_count, sizeof(int), hipMemcpyDeviceToHost, st));
    VQ_HIP(hipStreamSynchronize(st));
    (void)n_sub;
    return VQ_OK;
}

}  // namespace vq
