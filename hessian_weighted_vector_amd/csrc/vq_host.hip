// Host side of libvq: the C ABI entry points (argument validation, workspace
// carving, launches), the codebook seeding walk and the whole-fit driver.
#include "vq_internal.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

namespace vq {

// ---- errors ---------------------------------------------------------------
namespace {
thread_local std::string g_err;
}

void set_error(const std::string& msg) { g_err = msg; }

vq_status fail(vq_status st, const std::string& msg)
{
    g_err = msg;
    return st;
}

vq_status hip_fail(hipError_t e, const char* what)
{
    g_err = std::string(what) + ": " + hipGetErrorString(e);
    return VQ_ERR_DEVICE;
}

// ---- launchers defined in the kernel files --------------------------------
vq_status assign_launch(const float*, const float*, const float*, const uint8_t*, int64_t, int64_t,
                        int, const float*, int, uint16_t*, float*, void*, size_t, hipStream_t);
vq_status assign_flag_count(void*, size_t, int64_t, int, int*, hipStream_t);
vq_status assign_flag_list(void*, size_t, int64_t, int, int32_t*, int64_t, int64_t*, hipStream_t);
size_t assign_scratch_bytes();
vq_status assign_noalloc_launch(const float*, const float*, const float*, const uint8_t*, int64_t, int64_t, int,
                                const float*, int, uint16_t*, float*, hipStream_t);
vq_status update_launch(const float*, const float*, const float*, const uint8_t*, int64_t, int64_t,
                        int, const uint16_t*, int, float*, int32_t*, void*, size_t, hipStream_t);
vq_status objective_launch(const float*, const float*, const float*, const uint8_t*, int64_t,
                           int64_t, int, const float*, int, const uint16_t*, double*, void*, size_t,
                           hipStream_t);
vq_status select_launch(const float*, const float*, int64_t, int64_t, int, int64_t, int32_t*,
                        int32_t*, float*, uint8_t*, void*, size_t, hipStream_t);
vq_status binorm_launch(const float*, const float*, int64_t, int64_t, float*, float*, float*,
                        float*, float*, void*, size_t, hipStream_t);
vq_status residual_launch(const float*, int64_t, int64_t, int, const float*, int, const uint16_t*,
                          float*, hipStream_t);
vq_status reconstruct_launch(int64_t, int64_t, int, const float*, int, const uint16_t*, const float*, int,
                             const uint16_t*, const float*, const float*, const int32_t*,
                             const int32_t*, const float*, float*, hipStream_t);
vq_status subvector_select_launch(const float*, const float*, int64_t, int64_t, int, int64_t, uint8_t*, void*,
                                  size_t, hipStream_t);
vq_status residual_select_launch(const float*, const float*, const float*, int64_t, int64_t, int, int64_t,
                                 uint8_t*, void*, size_t, hipStream_t);
vq_status mask_to_csr_launch(const float*, const uint8_t*, int64_t, int64_t, int, int64_t, int32_t*, int32_t*,
                             float*, void*, size_t, hipStream_t);
vq_status vptq_launch(const float*, const float*, int64_t, int64_t, int, const float*, int, int, uint16_t*, float*,
                      float*, void*, size_t, hipStream_t);
vq_status hfactor_launch(const float*, int64_t, double, float*, void*, size_t, hipStream_t);
vq_status sparse_overwrite_launch(int64_t, int64_t, const int32_t*, const int32_t*, const float*, float*,
                                  hipStream_t);
int column_order_slices(int64_t N);
vq_status column_order_launch(const float*, int64_t, int64_t, int32_t*, uint8_t*, int32_t*, hipStream_t);
vq_status gather_cols_launch(const float*, int64_t, int64_t, const int32_t*, int64_t, float*, hipStream_t);
vq_status scatter_cols_launch(const float*, int64_t, int64_t, const int32_t*, float*, int64_t, hipStream_t);
vq_status gather_mask_launch(const uint8_t*, int64_t, int64_t, int, const int32_t*, int64_t, int, uint8_t*,
                             hipStream_t);
vq_status qgemv_launch(int64_t, int64_t, int, const float*, int, const uint16_t*, const float*, int,
                       const uint16_t*, const float*, const float*, const int32_t*, const int32_t*,
                       const float*, const float*, int64_t, float*, void*, size_t, hipStream_t);

// ---- validation -------------------------------------------------------------
vq_status check_shape(int64_t M, int64_t N, int d)
{
    if (M <= 0 || N <= 0) return fail(VQ_ERR_INVALID, "M and N must be positive");
    if (d < 1 || d > 8) return fail(VQ_ERR_INVALID, "d must be in [1, 8]");
    if (N % d != 0) return fail(VQ_ERR_INVALID, "N must be a multiple of d");
    if (M > INT32_MAX || N > INT32_MAX || M * N / d > (int64_t)INT32_MAX || M * N > ((int64_t)1 << 40))
        return fail(VQ_ERR_INVALID, "matrix too large (sub-vector count must fit int32)");
    return VQ_OK;
}

vq_status check_K(int K, int64_t n_sub)
{
    if (K < 1 || K > 65536) return fail(VQ_ERR_INVALID, "K must be in [1, 65536]");
    if ((int64_t)K > n_sub) return fail(VQ_ERR_INVALID, "K exceeds the number of sub-vectors");
    return VQ_OK;
}

namespace {

#define VQ_WS(cond, msg)                                            \
    do {                                                          \
        if (!(cond)) return ::vq::fail(VQ_ERR_WORKSPACE, (msg));  \
    } while (0)

#define VQ_TRY(expr)                          \
    do {                                      \
        vq_status vq_s_ = (expr);             \
        if (vq_s_ != VQ_OK) return vq_s_;     \
    } while (0)

// VQ_CHECK=1 mode: finite values (weights: also non-negative) in an input.
#define VQ_VALUES(a, n, weights, call, what) \
    VQ_TRY(::vq::check_values((a), (n), (weights), (call), (what), as_stream(stream)))

// The current device must be a gfx950; checked once per device.
vq_status check_device()
{
    int dev = -1;
    VQ_HIP(hipGetDevice(&dev));
    static thread_local int ok_dev = -1;
    if (ok_dev == dev) return VQ_OK;
    hipDeviceProp_t prop;
    VQ_HIP(hipGetDeviceProperties(&prop, dev));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(VQ_ERR_UNSUPPORTED, std::string("libvq needs a gfx950 device, found ") + prop.gcnArchName);
    ok_dev = dev;
    return VQ_OK;
}

int64_t nnz_of(int64_t M, int64_t N, double p) { return (int64_t)std::floor(p * (double)(M * N)); }

constexpr int64_t kInitChunkMin = 65536;

int64_t init_chunk(int64_t n_sub, int K) { return std::min<int64_t>(n_sub, std::max<int64_t>(2 * (int64_t)K, kInitChunkMin)); }

// Slots of the device table for one chunk: a power of two, at least twice the chunk.
int64_t init_table_cap(int64_t chunk)
{
    int64_t cap = 16;
    while (cap < 2 * chunk) cap <<= 1;
    return cap;
}

// Gathers the chunk's candidate sub-vectors in walk order.
__global__ void k_gather(const float* __restrict__ X, const int32_t* __restrict__ perm, int64_t n, int d,
                         float* __restrict__ out)
{
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= n * d) return;
    const int64_t q = e / d;
    const int t = (int)(e - q * d);
    out[e] = X[(int64_t)perm[q] * d + t];
}

// Bitwise-distinct rows of the gathered chunk, on the device: an
// open-addressing table keyed by the row's bits keeps, per distinct value,
// the smallest walk position holding it (positions only ever go down, and a
// slot's value never changes once claimed), so the outcome does not depend on
// the order in which threads arrive.  A position is taken when it is the
// first of its value; positions keep walk order through a block-wise scan.
constexpr int kInitThreads = 1024;
constexpr int32_t kInitEmpty = 0x7FFFFFFF;

__device__ inline uint32_t row_hash(const uint32_t (&w)[8], int d)
{
    uint64_t hsh = 0x9E3779B97F4A7C15ull ^ (uint64_t)d;
    for (int t = 0; t < d; ++t) {
        hsh += w[t];
        hsh ^= hsh >> 30;
        hsh *= 0xBF58476D1CE4E5B9ull;
        hsh ^= hsh >> 27;
        hsh *= 0x94D049BB133111EBull;
        hsh ^= hsh >> 31;
    }
    return (uint32_t)hsh;
}

__device__ inline void load_row_bits(const float* __restrict__ rows, int64_t q, int d, uint32_t (&w)[8])
{
#pragma unroll
    for (int t = 0; t < 8; ++t) w[t] = t < d ? __float_as_uint(rows[q * d + t]) : 0u;
}

__device__ inline bool row_equal(const float* __restrict__ rows, int64_t r, int d, const uint32_t (&w)[8])
{
    for (int t = 0; t < d; ++t)
        if (__float_as_uint(rows[r * d + t]) != w[t]) return false;
    return true;
}

__global__ __launch_bounds__(256) void k_init_fill(int32_t* __restrict__ table, int64_t cap)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q < cap) table[q] = kInitEmpty;
}

__global__ __launch_bounds__(256) void k_init_insert(const float* __restrict__ rows, int64_t n, int d,
                                                     int32_t* __restrict__ table, uint32_t cap_mask)
{
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= n) return;
    uint32_t w[8];
    load_row_bits(rows, q, d, w);
    uint32_t h = row_hash(w, d) & cap_mask;
    for (;;) {
        int32_t r = __atomic_load_n(&table[h], __ATOMIC_RELAXED);
        if (r == kInitEmpty) {
            r = atomicCAS(&table[h], kInitEmpty, (int32_t)q);
            if (r == kInitEmpty) return;
        }
        if (row_equal(rows, r, d, w)) {
            atomicMin(&table[h], (int32_t)q);
            return;
        }
        h = (h + 1) & cap_mask;
    }
}

// flag[q] = 1 when q is the first position of its value; per-block counts.
__global__ __launch_bounds__(kInitThreads) void k_init_flag(const float* __restrict__ rows, int64_t n, int d,
                                                            const int32_t* __restrict__ table, uint32_t cap_mask,
                                                            int32_t* __restrict__ flag, int32_t* __restrict__ bcount)
{
    __shared__ int wsum[kInitThreads / 64];
    const int64_t q = (int64_t)blockIdx.x * kInitThreads + threadIdx.x;
    int f = 0;
    if (q < n) {
        uint32_t w[8];
        load_row_bits(rows, q, d, w);
        uint32_t h = row_hash(w, d) & cap_mask;
        for (;;) {
            const int32_t r = table[h];
            if (r != kInitEmpty && row_equal(rows, r, d, w)) {
                f = r == (int32_t)q;
                break;
            }
            h = (h + 1) & cap_mask;
        }
        flag[q] = f;
    }
    const unsigned long long b = __ballot(f);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = __popcll(b);
    __syncthreads();
    if (threadIdx.x == 0) {
        int c = 0;
        for (int k = 0; k < kInitThreads / 64; ++k) c += wsum[k];
        bcount[blockIdx.x] = c;
    }
}

// Exclusive scan of the block counts (one block); boff[nblk] = total.
__global__ __launch_bounds__(256) void k_init_scan(const int32_t* __restrict__ bcount, int nblk,
                                                   int32_t* __restrict__ boff)
{
    if (threadIdx.x != 0) return;
    int run = 0;
    for (int k = 0; k < nblk; ++k) {
        boff[k] = run;
        run += bcount[k];
    }
    boff[nblk] = run;
}

// The first K taken positions, in walk order, become the codebook rows.
__global__ __launch_bounds__(kInitThreads) void k_init_write(const float* __restrict__ rows, int64_t n, int d,
                                                             const int32_t* __restrict__ flag,
                                                             const int32_t* __restrict__ boff, int K,
                                                             float* __restrict__ C)
{
    __shared__ int wsum[kInitThreads / 64];
    const int64_t q = (int64_t)blockIdx.x * kInitThreads + threadIdx.x;
    const int f = q < n ? flag[q] : 0;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const unsigned long long b = __ballot(f);
    if (lane == 0) wsum[wave] = __popcll(b);
    __syncthreads();
    int pos = boff[blockIdx.x] + __popcll(b & ((1ull << lane) - 1ull));
    for (int k = 0; k < wave; ++k) pos += wsum[k];
    if (f && pos < K)
        for (int t = 0; t < d; ++t) C[(int64_t)pos * d + t] = rows[q * d + t];
}

uint64_t mix64(const uint32_t* w, int d)
{
    uint64_t hsh = 0x9E3779B97F4A7C15ull ^ (uint64_t)d;
    for (int t = 0; t < d; ++t) {
        hsh += w[t];
        hsh ^= hsh >> 30;
        hsh *= 0xBF58476D1CE4E5B9ull;
        hsh ^= hsh >> 27;
        hsh *= 0x94D049BB133111EBull;
        hsh ^= hsh >> 31;
    }
    return hsh;
}

// The seeding walk: first K bitwise-distinct sub-vectors in perm order.
vq_status init_walk(const float* X, int64_t n_sub, int d, const int32_t* perm, int K, float* C,
                    void* ws, size_t ws_bytes, hipStream_t st)
{
    const int64_t chunk = init_chunk(n_sub, K);
    Carver cv(ws, ws_bytes);
    int32_t* dperm = cv.take<int32_t>(chunk);
    float* dbuf = cv.take<float>((size_t)chunk * d);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_init: workspace too small");

    TimedRegion tr("init", K, st);
    {
        // the first chunk on the device; if it holds fewer than K distinct
        // rows, the walk is done again below on the host, chunk by chunk
        const int64_t n = chunk;
        for (int64_t q = 0; q < n; ++q)
            if (perm[q] < 0 || perm[q] >= n_sub) return fail(VQ_ERR_INVALID, "perm holds an id outside [0, n_sub)");
        const int64_t cap = init_table_cap(chunk);
        const int nblk = (int)((n + kInitThreads - 1) / kInitThreads);
        int32_t* table = cv.take<int32_t>((size_t)cap);
        int32_t* flag = cv.take<int32_t>((size_t)chunk);
        int32_t* bcount = cv.take<int32_t>((size_t)nblk);
        int32_t* boff = cv.take<int32_t>((size_t)nblk + 1);
        if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_init: workspace too small");
        VQ_HIP(hipMemcpyAsync(dperm, perm, (size_t)n * sizeof(int32_t), hipMemcpyHostToDevice, st));
        hipLaunchKernelGGL(k_gather, dim3(grid_for(n * d, 256)), dim3(256), 0, st, X, dperm, n, d, dbuf);
        VQ_LAUNCHED("k_gather");
        hipLaunchKernelGGL(k_init_fill, dim3(grid_for(cap, 256)), dim3(256), 0, st, table, cap);
        VQ_LAUNCHED("k_init_fill");
        hipLaunchKernelGGL(k_init_insert, dim3(grid_for(n, 256)), dim3(256), 0, st, dbuf, n, d, table,
                           (uint32_t)(cap - 1));
        VQ_LAUNCHED("k_init_insert");
        hipLaunchKernelGGL(k_init_flag, dim3(nblk), dim3(kInitThreads), 0, st, dbuf, n, d, table,
                           (uint32_t)(cap - 1), flag, bcount);
        VQ_LAUNCHED("k_init_flag");
        hipLaunchKernelGGL(k_init_scan, dim3(1), dim3(256), 0, st, bcount, nblk, boff);
        VQ_LAUNCHED("k_init_scan");
        hipLaunchKernelGGL(k_init_write, dim3(nblk), dim3(kInitThreads), 0, st, dbuf, n, d, flag, boff, K, C);
        VQ_LAUNCHED("k_init_write");
        int32_t total = 0;
        VQ_HIP(hipMemcpyAsync(&total, boff + nblk, sizeof(int32_t), hipMemcpyDeviceToHost, st));
        VQ_HIP(hipStreamSynchronize(st));
        if (total >= K) return VQ_OK;
    }
    std::vector<float> host((size_t)chunk * d);
    std::vector<float> taken_rows((size_t)K * d);
    size_t cap = 16;
    while (cap < (size_t)K * 2 + 2) cap <<= 1;
    std::vector<int32_t> table(cap, -1);
    int taken = 0;
    for (int64_t e0 = 0; e0 < n_sub && taken < K; e0 += chunk) {
        const int64_t n = std::min<int64_t>(chunk, n_sub - e0);
        for (int64_t q = 0; q < n; ++q)
            if (perm[e0 + q] < 0 || perm[e0 + q] >= n_sub)
                return fail(VQ_ERR_INVALID, "perm holds an id outside [0, n_sub)");
        VQ_HIP(hipMemcpyAsync(dperm, perm + e0, (size_t)n * sizeof(int32_t), hipMemcpyHostToDevice, st));
        hipLaunchKernelGGL(k_gather, dim3(grid_for(n * d, 256)), dim3(256), 0, st, X, dperm, n, d, dbuf);
        VQ_LAUNCHED("k_gather");
        VQ_HIP(hipMemcpyAsync(host.data(), dbuf, (size_t)n * d * sizeof(float), hipMemcpyDeviceToHost, st));
        VQ_HIP(hipStreamSynchronize(st));
        for (int64_t q = 0; q < n && taken < K; ++q) {
            const float* v = host.data() + (size_t)q * d;
            uint32_t w[8];
            std::memcpy(w, v, sizeof(float) * d);
            size_t pos = (size_t)(mix64(w, d) & (cap - 1));
            bool dup = false;
            while (table[pos] >= 0) {
                if (std::memcmp(taken_rows.data() + (size_t)table[pos] * d, v, sizeof(float) * d) == 0) {
                    dup = true;
                    break;
                }
                pos = (pos + 1) & (cap - 1);
            }
            if (dup) continue;
            std::memcpy(taken_rows.data() + (size_t)taken * d, v, sizeof(float) * d);
            table[pos] = taken++;
        }
    }
    if (taken < K)
        return fail(VQ_ERR_INIT, "only " + std::to_string(taken) + " distinct sub-vectors, K = " + std::to_string(K));
    VQ_HIP(hipMemcpyAsync(C, taken_rows.data(), (size_t)K * d * sizeof(float), hipMemcpyHostToDevice, st));
    VQ_HIP(hipStreamSynchronize(st));
    return VQ_OK;
}

size_t ws_update_total(int64_t n_sub, int K) { return ws_objective(n_sub) + ws_update(n_sub, K); }

// Objective then update, each with its own slice of the workspace.
vq_status update_with_J(const float* X, const float* hcol, const float* rho, const uint8_t* mask, int64_t M,
                        int64_t N, int d, const uint16_t* idx, int K, float* C, int32_t* counts,
                        double* J, void* ws, size_t ws_bytes, hipStream_t st)
{
    const int64_t n_sub = M * N / d;
    const size_t wo = ws_objective(n_sub);
    if (ws_bytes < wo) return fail(VQ_ERR_WORKSPACE, "vq_update: workspace too small");
    if (J) VQ_TRY(objective_launch(X, hcol, rho, mask, M, N, d, C, K, idx, J, ws, wo, st));
    return update_launch(X, hcol, rho, mask, M, N, d, idx, K, C, counts, static_cast<char*>(ws) + wo,
                         ws_bytes - wo, st);
}

// Centroids with no member: one workgroup of 1024 counts the zero entries
// of counts[0..K) (16-byte loads when K % 4 == 0 and the array allows, a
// wavefront butterfly, the 16 wavefront sums in order: an exact integer
// count) and writes the total to *out.
__global__ __launch_bounds__(1024) void k_count_empty(const int32_t* __restrict__ counts, int K,
                                                      unsigned long long* __restrict__ out)
{
    __shared__ unsigned ws16[16];
    unsigned c = 0;
    if ((K & 3) == 0 && (reinterpret_cast<uintptr_t>(counts) & 15u) == 0) {
        const int4* c4 = reinterpret_cast<const int4*>(counts);
#pragma unroll 4
        for (int i = threadIdx.x; i < K / 4; i += 1024) {
            const int4 v = c4[i];
            c += (v.x == 0) + (v.y == 0) + (v.z == 0) + (v.w == 0);
        }
    } else {
        for (int k = threadIdx.x; k < K; k += 1024) c += counts[k] == 0 ? 1u : 0u;
    }
    for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
    if ((threadIdx.x & 63) == 0) ws16[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned long long t = 0;
        for (int w = 0; w < 16; ++w) t += ws16[w];
        *out = t;
    }
}

// One Lloyd stage: T x (assign, objective, update), final assign, objective.
// With emp: the update also counts members (into counts[K]) and emp[t]
// receives the number of centroids left with none.
vq_status lloyd_stage(const float* X, const float* hcol, const float* rho, const uint8_t* mask, int64_t M,
                      int64_t N, int d, float* C, int K, int T, uint16_t* idx, double* Jd, void* ws,
                      size_t ws_bytes, hipStream_t st, int32_t* counts = nullptr,
                      unsigned long long* emp = nullptr)
{
    for (int t = 0; t < T; ++t) {
        VQ_TRY(assign_launch(X, hcol, rho, mask, M, N, d, C, K, idx, nullptr, ws, ws_bytes, st));
        VQ_TRY(update_with_J(X, hcol, rho, mask, M, N, d, idx, K, C, emp ? counts : nullptr, Jd + t, ws, ws_bytes,
                             st));
        if (emp) {
            hipLaunchKernelGGL(k_count_empty, dim3(1), dim3(1024), 0, st, counts, K, emp + t);
            VQ_LAUNCHED("k_count_empty");
        }
    }
    VQ_TRY(assign_launch(X, hcol, rho, mask, M, N, d, C, K, idx, nullptr, ws, ws_bytes, st));
    return objective_launch(X, hcol, rho, mask, M, N, d, C, K, idx, Jd + T, ws, ws_bytes, st);
}

size_t ws_steps(int64_t M, int64_t N, int d, int K1, int K2)
{
    const int64_t n_sub = M * N / d;
    const int Kmax = std::max(K1, K2);
    // the assignment with its optional arrays (two-pass search, chunk path)
    size_t w = ws_assign_full(n_sub, Kmax);
    // the update's needs are not monotone in K (a short codebook takes more
    // pieces, a long one the bucket arrays): both stages' sizes
    w = std::max(w, ws_update_total(n_sub, K1));
    w = std::max(w, ws_update_total(n_sub, K2));
    w = std::max(w, ws_select(M, N));
    w = std::max(w, ws_binorm(M, N));
    w = std::max(w, ws_init(n_sub, Kmax, d));
    return w;
}

}  // namespace

size_t ws_init(int64_t n_sub, int K, int d)
{
    const int64_t chunk = init_chunk(n_sub, K);
    const int64_t nblk = (chunk + kInitThreads - 1) / kInitThreads;
    return align_up((size_t)chunk * sizeof(int32_t)) + align_up((size_t)chunk * d * sizeof(float)) +
           align_up((size_t)init_table_cap(chunk) * sizeof(int32_t)) + align_up((size_t)chunk * sizeof(int32_t)) +
           align_up((size_t)nblk * sizeof(int32_t)) + align_up((size_t)(nblk + 1) * sizeof(int32_t));
}

}  // namespace vq

using namespace vq;

// ============================================================================
extern "C" {

const char* vq_version(void) { return "libvq 0.1.0 (gfx950)"; }

const char* vq_last_error(void) { return g_err.c_str(); }

size_t vq_workspace_bytes(int64_t M, int64_t N, int d, int K1, int K2, int64_t nnz)
{
    (void)nnz;
    if (M <= 0 || N <= 0 || d < 1 || d > 8 || N % d) return 0;
    const int64_t n_sub = M * N / d;
    const int iters_guess = 256;   // J history slots reserved in the workspace
    size_t w = ws_steps(M, N, d, std::max(K1, 1), std::max(K2, 1));
    if (K2 > 0) w += align_up((size_t)M * N * sizeof(float));
    w += align_up(sizeof(double) * iters_guess);
    w += align_up(sizeof(int32_t) * (size_t)std::max(std::max(K1, K2), 1));   // member counts
    w += align_up(sizeof(unsigned long long) * iters_guess);                  // empty-centroid history
    (void)n_sub;
    return w;
}

vq_status vq_sparse_select(const float* W, const float* h, int64_t M, int64_t N, int d, int64_t nnz,
                           int32_t* row_ptr, int32_t* col, float* val, uint8_t* mask, void* ws,
                           size_t ws_bytes, void* stream)
{
    VQ_TRY(check_shape(M, N, d));
    VQ_CHECK(W && h && row_ptr && mask, "vq_sparse_select: null pointer");
    VQ_CHECK(nnz >= 0 && nnz <= M * N && nnz <= INT32_MAX, "vq_sparse_select: nnz out of range");
    VQ_CHECK(nnz == 0 || (col && val), "vq_sparse_select: col/val are null");
    VQ_WS(ws_bytes >= ws_select(M, N) && ws, "vq_sparse_select: workspace too small");
    VQ_TRY(check_device());
    VQ_VALUES(W, M * N, false, "vq_sparse_select", "W");
    VQ_VALUES(h, N, true, "vq_sparse_select", "h");
    return select_launch(W, h, M, N, d, nnz, row_ptr, col, val, mask, ws, ws_bytes, as_stream(stream));
}

vq_status vq_binorm(const float* W, const float* h, int64_t M, int64_t N, float* Wp, float* r, float* c,
                    float* hcol, float* rho, void* ws, size_t ws_bytes, void* stream)
{
    VQ_TRY(check_shape(M, N, 1));
    VQ_CHECK(W && h && Wp && r && c && hcol && rho, "vq_binorm: null pointer");
    VQ_CHECK(Wp != W, "vq_binorm: Wp may not alias W");
    VQ_WS(ws && ws_bytes >= ws_binorm(M, N), "vq_binorm: workspace too small");
    VQ_TRY(check_device());
    VQ_VALUES(W, M * N, false, "vq_binorm", "W");
    VQ_VALUES(h, N, true, "vq_binorm", "h");
    return binorm_launch(W, h, M, N, Wp, r, c, hcol, rho, ws, ws_bytes, as_stream(stream));
}

vq_status vq_init(const float* X, int64_t M, int64_t N, int d, const int32_t* perm, int K, float* C,
                  void* ws, size_t ws_bytes, void* stream)
{
    VQ_TRY(check_shape(M, N, d));
    const int64_t n_sub = M * N / d;
    VQ_TRY(check_K(K, n_sub));
    VQ_CHECK(X && perm && C, "vq_init: null pointer");
    VQ_WS(ws && ws_bytes >= ws_init(n_sub, K, d), "vq_init: workspace too small");
    VQ_TRY(check_device());
    VQ_VALUES(X, M * N, false, "vq_init", "X");
    return init_walk(X, n_sub, d, perm, K, C, ws, ws_bytes, as_stream(stream));
}

vq_status vq_assign(const float* X, const float* hcol, const float* rho, const uint8_t* mask, int64_t M,
                    int64_t N, int d, const float* C, int K, uint16_t* idx, float* dist, void* ws,
                    size_t ws_bytes, void* stream)
{
    VQ_TRY(check_shape(M, N, d));
    const int64_t n_sub = M * N / d;
    VQ_TRY(check_K(K, n_sub));
    VQ_CHECK(X && hcol && C && idx, "vq_assign: null pointer");
    VQ_WS(ws && ws_bytes >= ws_assign(n_sub, K), "vq_assign: workspace too small");
    VQ_TRY(check_device());
    VQ_VALUES(X, M * N, false, "vq_assign", "X");
    VQ_VALUES(hcol, N, true, "vq_assign", "hcol");
    VQ_VALUES(rho, M, true, "vq_assign", "rho");
    VQ_VALUES(C, (int64_t)K * d, false, "vq_assign", "C");
    return assign_launch(X, hcol, rho, mask, M, N, d, C, K, idx, dist, ws, ws_bytes, as_stream(stream));
}

vq_status vq_assign_noalloc(const float* X, const float* hcol, const float* rho, const uint8_t* mask, int64_t M,
                            int64_t N, int d, const float* C, int K, uint16_t* idx, float* dist, void* stream)
{
    VQ_TRY(check_shape(M, N, d));
    const int64_t n_sub = M * N / d;
    VQ_TRY(check_K(K, n_sub));
    VQ_CHECK(X && hcol && C && idx, "vq_assign_noalloc: null pointer");
    const size_t need = ws_assign(n_sub, K);
    if (need > assign_scratch_bytes())
        return fail(VQ_ERR_INVALID, "vq_assign_noalloc: these sizes need " + std::to_string(need) +
                                        " bytes of scratch; the library holds " +
                                        std::to_string(assign_scratch_bytes()) + " per device");
    VQ_TRY(check_device());
    VQ_VALUES(X, M * N, false, "vq_assign_noalloc", "X");
    VQ_VALUES(hcol, N, true, "vq_assign_noalloc", "hcol");
    VQ_VALUES(rho, M, true, "vq_assign_noalloc", "rho");
    VQ_VALUES(C, (int64_t)K * d, false, "vq_assign_noalloc", "C");
    return assign_noalloc_launch(X, hcol, rho, mask, M, N, d, C, K, idx, dist, as_stream(stream));
}

vq_status vq_update(const float* X, const float* hcol, const float* rho, const uint8_t* mask, int64_t M,
                    int64_t N, int d, const uint16_t* idx, int K, float* C, int32_t* counts, double* J,
                    void* ws, size_t ws_bytes, void* stream)
{
    VQ_TRY(check_shape(M, N, d));
    const int64_t n_sub = M * N / d;
    VQ_TRY(check_K(K, n_sub));
    VQ_CHECK(X && hcol && idx && C, "vq_update: null pointer");
    VQ_WS(ws && ws_bytes >= ws_update_total(n_sub, K), "vq_update: workspace too small");
    VQ_TRY(check_device());
    VQ_VALUES(X, M * N, false, "vq_update", "X");
    VQ_VALUES(hcol, N, true, "vq_update", "hcol");
    VQ_VALUES(rho, M, true, "vq_update", "rho");
    VQ_VALUES(C, (int64_t)K * d, false, "vq_update", "C");
    return update_with_J(X, hcol, rho, mask, M, N, d, idx, K, C, counts, J, ws, ws_bytes, as_stream(stream));
}

vq_status vq_objective(const float* X, const float* hcol, const float* rho, const uint8_t* mask, int64_t M,
                       int64_t N, int d, const float* C, int K, const uint16_t* idx, double* J, void* ws,
                       size_t ws_bytes, void* stream)
{
    VQ_TRY(check_shape(M, N, d));
    const int64_t n_sub = M * N / d;
    VQ_TRY(check_K(K, n_sub));
    VQ_CHECK(X && hcol && C && idx && J, "vq_objective: null pointer");
    VQ_WS(ws && ws_bytes >= ws_objective(n_sub), "vq_objective: workspace too small");
    VQ_TRY(check_device());
    VQ_VALUES(X, M * N, false, "vq_objective", "X");
    VQ_VALUES(hcol, N, true, "vq_objective", "hcol");
    VQ_VALUES(rho, M, true, "vq_objective", "rho");
    VQ_VALUES(C, (int64_t)K * d, false, "vq_objective", "C");
    return objective_launch(X, hcol, rho, mask, M, N, d, C, K, idx, J, ws, ws_bytes, as_stream(stream));
}

vq_status vq_residual(const float* X, int64_t M, int64_t N, int d, const float* C, int K, const uint16_t* idx,
                      float* R, void* stream)
{
    VQ_TRY(check_shape(M, N, d));
    VQ_TRY(check_K(K, M * N / d));
    VQ_CHECK(X && C && idx && R, "vq_residual: null pointer");
    VQ_CHECK(R != X, "vq_residual: R may not alias X");
    VQ_TRY(check_device());
    VQ_VALUES(X, M * N, false, "vq_residual", "X");
    VQ_VALUES(C, (int64_t)K * d, false, "vq_residual", "C");
    return residual_launch(X, M, N, d, C, K, idx, R, as_stream(stream));
}

vq_status vq_reconstruct(int64_t M, int64_t N, int d, const float* C1, int K1, const uint16_t* idx1,
                         const float* C2, int K2, const uint16_t* idx2, const float* rscale, const float* cscale,
                         const int32_t* row_ptr, const int32_t* col, const float* val, float* W_hat, void* stream)
{
    VQ_TRY(check_shape(M, N, d));
    const int64_t n_sub = M * N / d;
    VQ_TRY(check_K(K1, n_sub));
    VQ_CHECK(C1 && idx1 && W_hat, "vq_reconstruct: null pointer");
    if (C2) {
        VQ_TRY(check_K(K2, n_sub));
        VQ_CHECK(idx2 != nullptr, "vq_reconstruct: idx2 is null");
    }
    VQ_CHECK(!row_ptr || (col && val), "vq_reconstruct: col/val are null");
    VQ_TRY(check_device());
    VQ_VALUES(C1, (int64_t)K1 * d, false, "vq_reconstruct", "C1");
    VQ_VALUES(C2, (int64_t)K2 * d, false, "vq_reconstruct", "C2");
    VQ_VALUES(rscale, M, false, "vq_reconstruct", "rscale");
    VQ_VALUES(cscale, N, false, "vq_reconstruct", "cscale");
    return reconstruct_launch(M, N, d, C1, K1, idx1, C2, K2, idx2, rscale, cscale, row_ptr, col, val, W_hat,
                              as_stream(stream));
}

vq_status vq_select_subvectors(const float* W, const float* h, int64_t M, int64_t N, int d, int64_t n_sel,
                               uint8_t* mask, void* ws, size_t ws_bytes, void* stream)
{
    VQ_TRY(check_shape(M, N, d));
    const int64_t n_sub = M * N / d;
    VQ_CHECK(W && h && mask, "vq_select_subvectors: null pointer");
    VQ_CHECK(n_sel >= 0 && n_sel <= n_sub, "vq_select_subvectors: n_sel must be in [0, n_sub]");
    VQ_CHECK(n_sub <= (int64_t)UINT32_MAX, "vq_select_subvectors: too many sub-vectors");
    VQ_WS(ws && ws_bytes >= ws_select(M, N), "vq_select_subvectors: workspace too small");
    VQ_TRY(check_device());
    VQ_VALUES(W, M * N, false, "vq_select_subvectors", "W");
    VQ_VALUES(h, N, true, "vq_select_subvectors", "h");
    return subvector_select_launch(W, h, M, N, d, n_sel, mask, ws, ws_bytes, as_stream(stream));
}

vq_status vq_select_residual(const float* W, const float* W_hat, const float* h, int64_t M, int64_t N, int d,
                             int64_t n_sel, uint8_t* mask, void* ws, size_t ws_bytes, void* stream)
{
    VQ_TRY(check_shape(M, N, d));
    VQ_CHECK(W && W_hat && h && mask, "vq_select_residual: null pointer");
    VQ_CHECK(n_sel >= 0, "vq_select_residual: n_sel must be >= 0");
    VQ_CHECK(M * N / d <= (int64_t)UINT32_MAX, "vq_select_residual: too many sub-vectors");
    VQ_WS(ws && ws_bytes >= ws_select(M, N), "vq_select_residual: workspace too small");
    VQ_TRY(check_device());
    VQ_VALUES(W, M * N, false, "vq_select_residual", "W");
    VQ_VALUES(W_hat, M * N, false, "vq_select_residual", "W_hat");
    VQ_VALUES(h, N, true, "vq_select_residual", "h");
    return residual_select_launch(W, W_hat, h, M, N, d, n_sel, mask, ws, ws_bytes, as_stream(stream));
}

vq_status vq_mask_to_csr(const float* W, const uint8_t* mask, int64_t M, int64_t N, int d, int64_t nnz_cap,
                         int32_t* row_ptr, int32_t* col, float* val, void* ws, size_t ws_bytes, void* stream)
{
    VQ_TRY(check_shape(M, N, d));
    VQ_CHECK(W && mask && row_ptr, "vq_mask_to_csr: null pointer");
    VQ_CHECK(nnz_cap >= 0, "vq_mask_to_csr: nnz_cap must be >= 0");
    VQ_CHECK(nnz_cap == 0 || (col && val), "vq_mask_to_csr: col/val are null");
    VQ_CHECK(M * N <= (int64_t)INT32_MAX, "vq_mask_to_csr: M*N exceeds the int32 row pointer");
    VQ_WS(ws && ws_bytes >= ws_select(M, N), "vq_mask_to_csr: workspace too small");
    VQ_TRY(check_device());
    VQ_VALUES(W, M * N, false, "vq_mask_to_csr", "W");
    return mask_to_csr_launch(W, mask, M, N, d, nnz_cap, row_ptr, col, val, ws, ws_bytes, as_stream(stream));
}

size_t vq_hessian_factor_workspace_bytes(int64_t N)
{
    if (N <= 0) return 0;
    return ws_hfactor(N);
}

vq_status vq_hessian_factor(const float* H, int64_t N, double damp, float* U, void* ws, size_t ws_bytes,
                            void* stream)
{
    VQ_CHECK(N > 0 && N <= 65536, "vq_hessian_factor: N must be in [1, 65536]");
    VQ_CHECK(damp >= 0.0 && damp < 1e300, "vq_hessian_factor: damp must be finite and >= 0");
    VQ_CHECK(H && U && (const void*)H != (const void*)U, "vq_hessian_factor: null or aliased pointer");
    VQ_WS(ws && ws_bytes >= ws_hfactor(N), "vq_hessian_factor: workspace too small");
    VQ_TRY(check_device());
    VQ_VALUES(H, N * N, false, "vq_hessian_factor", "H");
    return hfactor_launch(H, N, damp, U, ws, ws_bytes, as_stream(stream));
}

size_t vq_vptq_workspace_bytes(int64_t M, int64_t N, int V)
{
    if (M <= 0 || N <= 0 || V < 1 || V > 8 || M % V) return 0;
    return ws_vptq(M, N, V);
}

vq_status vq_vptq(const float* W, const float* U, int64_t M, int64_t N, int V, const float* C, int K, int B,
                  uint16_t* idx, float* W_hat, float* E, void* ws, size_t ws_bytes, void* stream)
{
    VQ_CHECK(M > 0 && N > 0, "vq_vptq: M and N must be positive");
    VQ_CHECK(V >= 1 && V <= 8 && M % V == 0, "vq_vptq: V must be in [1, 8] and divide M");
    VQ_CHECK(K >= 1 && K <= 65536, "vq_vptq: K must be in [1, 65536]");
    VQ_CHECK(B >= 1 && B <= 128, "vq_vptq: B must be in [1, 128]");
    VQ_CHECK(M <= (int64_t)32 * 65535 && N <= (int64_t)32 * 65535 && M / V <= (int64_t)INT32_MAX,
             "vq_vptq: matrix too large");
    VQ_CHECK(W && U && C && idx && W_hat, "vq_vptq: null pointer");
    VQ_CHECK(W_hat != W && (E == nullptr || (E != W && E != W_hat)), "vq_vptq: outputs may not alias");
    VQ_WS(ws && ws_bytes >= ws_vptq(M, N, V), "vq_vptq: workspace too small");
    VQ_TRY(check_device());
    VQ_VALUES(W, M * N, false, "vq_vptq", "W");
    VQ_VALUES(U, N * N, false, "vq_vptq", "U");
    VQ_VALUES(C, (int64_t)K * V, false, "vq_vptq", "C");
    return vptq_launch(W, U, M, N, V, C, K, B, idx, W_hat, E, ws, ws_bytes, as_stream(stream));
}

size_t vq_qgemv_workspace_bytes(int64_t M, int64_t N, int d, int64_t B)
{
    if (M <= 0 || N <= 0 || d < 1 || d > 8 || N % d || B < 0) return 0;
    return ws_qgemv(M, N, d, B);
}

vq_status vq_qgemv(int64_t M, int64_t N, int d, const float* C1, int K1, const uint16_t* idx1,
                   const float* C2, int K2, const uint16_t* idx2, const float* rscale, const float* cscale,
                   const int32_t* row_ptr, const int32_t* col, const float* val, const float* X, int64_t B,
                   float* Y, void* ws, size_t ws_bytes, void* stream)
{
    VQ_TRY(check_shape(M, N, d));
    const int64_t n_sub = M * N / d;
    VQ_TRY(check_K(K1, n_sub));
    VQ_CHECK(C1 && idx1, "vq_qgemv: null pointer");
    if (C2) {
        VQ_TRY(check_K(K2, n_sub));
        VQ_CHECK(idx2 != nullptr, "vq_qgemv: idx2 is null");
    }
    VQ_CHECK(!row_ptr || (col && val), "vq_qgemv: col/val are null");
    VQ_CHECK(B >= 0, "vq_qgemv: B must be >= 0");
    if (B == 0) return VQ_OK;
    VQ_CHECK(X && Y, "vq_qgemv: null pointer");
    VQ_CHECK((const void*)Y != (const void*)X, "vq_qgemv: Y may not alias X");
    const size_t need = ws_qgemv(M, N, d, B);
    VQ_WS(need == 0 || (ws && ws_bytes >= need), "vq_qgemv: workspace too small");
    VQ_TRY(check_device());
    VQ_VALUES(C1, (int64_t)K1 * d, false, "vq_qgemv", "C1");
    VQ_VALUES(C2, (int64_t)K2 * d, false, "vq_qgemv", "C2");
    VQ_VALUES(rscale, M, false, "vq_qgemv", "rscale");
    VQ_VALUES(cscale, N, false, "vq_qgemv", "cscale");
    VQ_VALUES(X, B * N, false, "vq_qgemv", "X");
    return qgemv_launch(M, N, d, C1, K1, idx1, C2, K2, idx2, rscale, cscale, row_ptr, col, val, X, B, Y, ws,
                        ws_bytes, as_stream(stream));
}

double vq_bits_per_weight(int64_t M, int64_t N, int d, int K1, int K2, int64_t nnz, int cb_bits, int binorm)
{
    if (M <= 0 || N <= 0 || d < 1 || N % d) return -1.0;
    auto ibits = [](int K) -> int64_t {
        int64_t b = 0;
        while (((int64_t)1 << b) < K) ++b;
        return b;
    };
    const int64_t n_sub = M * N / d;
    double bits = (double)n_sub * (double)(ibits(K1) + (K2 > 0 ? ibits(K2) : 0));
    bits += (double)d * (double)(K1 + (K2 > 0 ? K2 : 0)) * cb_bits;
    bits += 64.0 * (double)nnz;
    if (nnz > 0) bits += 32.0 * (double)(M + 1);
    if (binorm) bits += 32.0 * (double)(M + N);
    return bits / ((double)M * (double)N);
}

vq_status vq_fit(const vq_fit_params* p, const vq_fit_inputs* in, vq_fit_outputs* out, void* ws,
                 size_t ws_bytes, void* stream)
{
    VQ_CHECK(p && in && out, "vq_fit: null params/inputs/outputs");
    const int64_t M = p->M, N = p->N;
    const int d = p->d;
    VQ_TRY(check_shape(M, N, d));
    const int64_t n_sub = M * N / d;
    VQ_TRY(check_K(p->K1, n_sub));
    if (p->K2 > 0) VQ_TRY(check_K(p->K2, n_sub));
    VQ_CHECK(p->K2 >= 0, "vq_fit: K2 must be >= 0");
    VQ_CHECK(p->iters1 >= 0 && p->iters2 >= 0 && p->iters1 + p->iters2 + 2 <= 256, "vq_fit: iteration counts out of range");
    VQ_CHECK(p->outlier_frac >= 0.0 && p->outlier_frac <= 1.0, "vq_fit: outlier_frac must be in [0, 1]");
    const int64_t nnz = nnz_of(M, N, p->outlier_frac);
    VQ_CHECK(nnz <= INT32_MAX, "vq_fit: too many salient weights");
    VQ_CHECK(in->W && in->h, "vq_fit: W/h are null");
    VQ_CHECK(in->perm1 || in->C1_init, "vq_fit: need perm1 or C1_init");
    VQ_CHECK(p->K2 == 0 || in->perm2 || in->C2_init, "vq_fit: need perm2 or C2_init");
    VQ_CHECK(out->idx1 && out->C1 && out->row_ptr && out->mask && out->W_hat && out->J_hist,
             "vq_fit: null output");
    VQ_CHECK(nnz == 0 || (out->col && out->val), "vq_fit: col/val are null");
    VQ_CHECK(p->K2 == 0 || (out->idx2 && out->C2), "vq_fit: idx2/C2 are null");
    VQ_CHECK(!p->binorm || (out->Wp && out->rscale && out->cscale && out->hcol && out->rho),
             "vq_fit: bi-normalization outputs are null");
    const size_t need = vq_workspace_bytes(M, N, d, p->K1, p->K2, nnz);
    VQ_WS(ws && ws_bytes >= need, "vq_fit: workspace too small");
    VQ_TRY(check_device());
    VQ_VALUES(in->W, M * N, false, "vq_fit", "W");
    VQ_VALUES(in->h, N, true, "vq_fit", "h");
    VQ_VALUES(in->C1_init, (int64_t)p->K1 * d, false, "vq_fit", "C1_init");
    if (p->K2 > 0) VQ_VALUES(in->C2_init, (int64_t)p->K2 * d, false, "vq_fit", "C2_init");
    hipStream_t st = as_stream(stream);

    Carver cv(ws, ws_bytes);
    float* R = p->K2 > 0 ? cv.take<float>((size_t)M * N) : nullptr;
    double* Jd = cv.take<double>(256);
    int32_t* cnt = cv.take<int32_t>((size_t)std::max(std::max(p->K1, p->K2), 1));
    unsigned long long* emp = cv.take<unsigned long long>(256);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_fit: workspace too small");
    unsigned long long* emp_on = out->empty_hist ? emp : nullptr;
    void* sws = cv.base + cv.used;
    const size_t sws_bytes = cv.cap - cv.used;

    const float* X = in->W;
    const float* hc = in->h;
    const float* rh = nullptr;
    if (p->binorm) {
        VQ_TRY(binorm_launch(in->W, in->h, M, N, out->Wp, out->rscale, out->cscale, out->hcol, out->rho, sws,
                             sws_bytes, st));
        X = out->Wp;
        hc = out->hcol;
        rh = out->rho;
    }
    VQ_TRY(select_launch(in->W, in->h, M, N, d, nnz, out->row_ptr, out->col, out->val, out->mask, sws,
                         sws_bytes, st));
    const uint8_t* mk = p->mask_outliers ? out->mask : nullptr;

    if (in->C1_init)
        VQ_HIP(hipMemcpyAsync(out->C1, in->C1_init, (size_t)p->K1 * d * sizeof(float), hipMemcpyDeviceToDevice, st));
    else
        VQ_TRY(init_walk(X, n_sub, d, in->perm1, p->K1, out->C1, sws, sws_bytes, st));
    VQ_TRY(lloyd_stage(X, hc, rh, mk, M, N, d, out->C1, p->K1, p->iters1, out->idx1, Jd, sws, sws_bytes, st, cnt,
                       emp_on));
    const int nJ = p->iters1 + 1 + (p->K2 > 0 ? p->iters2 + 1 : 0);
    if (p->K2 > 0) {
        VQ_TRY(residual_launch(X, M, N, d, out->C1, p->K1, out->idx1, R, st));
        if (in->C2_init)
            VQ_HIP(hipMemcpyAsync(out->C2, in->C2_init, (size_t)p->K2 * d * sizeof(float), hipMemcpyDeviceToDevice, st));
        else
            VQ_TRY(init_walk(R, n_sub, d, in->perm2, p->K2, out->C2, sws, sws_bytes, st));
        VQ_TRY(lloyd_stage(R, hc, rh, mk, M, N, d, out->C2, p->K2, p->iters2, out->idx2, Jd + p->iters1 + 1, sws,
                           sws_bytes, st, cnt, emp_on ? emp_on + p->iters1 : nullptr));
    }
    VQ_TRY(reconstruct_launch(M, N, d, out->C1, p->K1, out->idx1, p->K2 > 0 ? out->C2 : nullptr, p->K2, out->idx2,
                              p->binorm ? out->rscale : nullptr, p->binorm ? out->cscale : nullptr,
                              nnz > 0 ? out->row_ptr : nullptr, out->col, out->val, out->W_hat, st));
    VQ_HIP(hipMemcpyAsync(out->J_hist, Jd, sizeof(double) * nJ, hipMemcpyDeviceToHost, st));
    const int nE = p->iters1 + (p->K2 > 0 ? p->iters2 : 0);
    if (emp_on && nE > 0)
        VQ_HIP(hipMemcpyAsync(out->empty_hist, emp, sizeof(int64_t) * nE, hipMemcpyDeviceToHost, st));
    VQ_HIP(hipStreamSynchronize(st));
    if (out->bpw) *out->bpw = vq_bits_per_weight(M, N, d, p->K1, p->K2, nnz, 32, p->binorm);
    return VQ_OK;
}

}  // extern "C"

namespace vq {
namespace {

struct GroupSpec {
    int64_t c0, Ng;   // first position in the column order, columns
    int d, K, T, K2, T2;
};

// Groups in order (outlier group first); false if the sizes do not split.
bool group_layout(const vq_grouped_params* p, std::vector<GroupSpec>& g)
{
    const vq_fit_params& f = p->fit;
    g.clear();
    if (f.N <= 0 || f.d < 1 || f.N % f.d || p->n_out < 0 || p->n_out % f.d || p->n_groups < 1) return false;
    if (p->n_out > 0) {
        if (p->d0 < 1 || p->d0 > 8 || p->n_out % p->d0) return false;
        g.push_back({0, p->n_out, p->d0, p->K0, p->iters0, 0, 0});
    }
    const int64_t nb = (f.N - p->n_out) / f.d;
    const int64_t w = (nb + p->n_groups - 1) / p->n_groups * f.d;
    if (nb < 1 || (int64_t)(p->n_groups - 1) * w >= f.N - p->n_out) return false;
    for (int q = 0; q < p->n_groups; ++q) {
        const int64_t c0 = p->n_out + q * w;
        g.push_back({c0, std::min(w, f.N - c0), f.d, f.K1, f.iters1, f.K2, f.iters2});
    }
    return true;
}

struct GroupTotals {
    int64_t n_idx = 0, n_cb = 0, n_J = 0, n_perm1 = 0, n_perm2 = 0, max_elems = 0, max_mask = 0;
    size_t steps = 0;
};

GroupTotals group_totals(const vq_grouped_params* p, const std::vector<GroupSpec>& g)
{
    GroupTotals t;
    const int64_t M = p->fit.M;
    for (const GroupSpec& s : g) {
        const int64_t ns = M * s.Ng / s.d;
        t.n_idx += ns * (s.K2 > 0 ? 2 : 1);
        t.n_cb += (int64_t)s.K * s.d + (int64_t)s.K2 * s.d;
        t.n_J += s.T + 1 + (s.K2 > 0 ? s.T2 + 1 : 0);
        t.n_perm1 += ns;
        if (s.K2 > 0) t.n_perm2 += ns;
        t.max_elems = std::max(t.max_elems, M * s.Ng);
        t.max_mask = std::max(t.max_mask, ns);
        t.steps = std::max(t.steps, ws_steps(M, s.Ng, s.d, s.K, s.K2));
    }
    t.steps = std::max(t.steps, std::max(ws_select(M, p->fit.N), ws_binorm(M, p->fit.N)));
    return t;
}

size_t grouped_ws(const vq_grouped_params* p, const GroupTotals& t)
{
    const int64_t M = p->fit.M, N = p->fit.N;
    size_t b = 0;
    if (p->fit.binorm)
        b += align_up((size_t)M * N * 4) + 2 * align_up((size_t)M * 4) + 2 * align_up((size_t)N * 4);
    b += 3 * align_up((size_t)t.max_elems * 4) + 2 * align_up((size_t)N * 4) + align_up((size_t)t.max_mask);
    b += align_up((size_t)N) + align_up((size_t)column_order_slices(N) * N * 4) + align_up((size_t)t.n_J * 8);
    return b + t.steps;
}

}  // namespace
}  // namespace vq

extern "C" {

double vq_bits_per_weight_grouped(const vq_grouped_params* p)
{
    std::vector<GroupSpec> g;
    if (!p || !group_layout(p, g) || p->fit.M <= 0) return -1.0;
    auto ibits = [](int K) -> int64_t {
        int64_t b = 0;
        while (((int64_t)1 << b) < K) ++b;
        return b;
    };
    const int64_t M = p->fit.M, N = p->fit.N;
    double bits = 0.0;
    for (const GroupSpec& s : g) {
        const double ns = (double)(M * s.Ng / s.d);
        bits += ns * (double)(ibits(s.K) + (s.K2 > 0 ? ibits(s.K2) : 0));
        bits += 32.0 * (double)s.d * (double)(s.K + (s.K2 > 0 ? s.K2 : 0));
    }
    const int64_t nnz = (int64_t)std::floor(p->fit.outlier_frac * (double)(M * N));
    bits += 64.0 * (double)nnz;
    if (nnz > 0) bits += 32.0 * (double)(M + 1);
    if (p->fit.binorm) bits += 32.0 * (double)(M + N);
    if (p->n_out > 0) bits += 32.0 * (double)p->n_out;
    return bits / ((double)M * (double)N);
}

size_t vq_grouped_sizes(const vq_grouped_params* p, int64_t* n_idx, int64_t* n_codebook, int64_t* n_J,
                        int64_t* n_perm1, int64_t* n_perm2)
{
    std::vector<GroupSpec> g;
    if (!p || !group_layout(p, g)) return 0;
    const GroupTotals t = group_totals(p, g);
    if (n_idx) *n_idx = t.n_idx;
    if (n_codebook) *n_codebook = t.n_cb;
    if (n_J) *n_J = t.n_J;
    if (n_perm1) *n_perm1 = t.n_perm1;
    if (n_perm2) *n_perm2 = t.n_perm2;
    return grouped_ws(p, t);
}

vq_status vq_fit_grouped(const vq_grouped_params* p, const vq_grouped_inputs* in, vq_grouped_outputs* out,
                         void* ws, size_t ws_bytes, void* stream)
{
    VQ_CHECK(p && in && out, "vq_fit_grouped: null params/inputs/outputs");
    const vq_fit_params& f = p->fit;
    const int64_t M = f.M, N = f.N;
    VQ_TRY(check_shape(M, N, f.d));
    std::vector<GroupSpec> groups;
    VQ_CHECK(group_layout(p, groups), "vq_fit_grouped: n_out must be a multiple of d and d0, and n_groups must "
                                      "split the other columns into non-empty groups");
    for (const GroupSpec& g : groups) {
        const int64_t ns = M * g.Ng / g.d;
        VQ_TRY(check_K(g.K, ns));
        if (g.K2 > 0) VQ_TRY(check_K(g.K2, ns));
    }
    VQ_CHECK(f.K2 >= 0 && f.iters1 >= 0 && f.iters2 >= 0 && p->iters0 >= 0, "vq_fit_grouped: negative count");
    VQ_CHECK(f.outlier_frac >= 0.0 && f.outlier_frac <= 1.0, "vq_fit_grouped: outlier_frac must be in [0, 1]");
    const int64_t nnz = nnz_of(M, N, f.outlier_frac);
    VQ_CHECK(nnz <= INT32_MAX, "vq_fit_grouped: too many salient weights");
    VQ_CHECK(in->W && in->h && in->perm1 && (f.K2 == 0 || in->perm2), "vq_fit_grouped: null input");
    VQ_CHECK(out->cols && out->idx && out->codebooks && out->row_ptr && out->mask && out->W_hat && out->J_hist,
             "vq_fit_grouped: null output");
    VQ_CHECK(nnz == 0 || (out->col && out->val), "vq_fit_grouped: col/val are null");
    const GroupTotals tot = group_totals(p, groups);
    VQ_WS(ws && ws_bytes >= grouped_ws(p, tot), "vq_fit_grouped: workspace too small");
    VQ_TRY(check_device());
    VQ_VALUES(in->W, p->fit.M * p->fit.N, false, "vq_fit_grouped", "W");
    VQ_VALUES(in->h, p->fit.N, true, "vq_fit_grouped", "h");
    hipStream_t st = as_stream(stream);

    Carver cv(ws, ws_bytes);
    float *Wp = nullptr, *r = nullptr, *c = nullptr, *hcol = nullptr, *rho = nullptr;
    if (f.binorm) {
        Wp = cv.take<float>((size_t)M * N);
        r = cv.take<float>(M);
        rho = cv.take<float>(M);
        c = cv.take<float>(N);
        hcol = cv.take<float>(N);
    }
    float* Xg = cv.take<float>(tot.max_elems);
    float* Rg = cv.take<float>(tot.max_elems);
    float* Wg = cv.take<float>(tot.max_elems);
    float* hg = cv.take<float>(N);
    float* cg = cv.take<float>(N);
    uint8_t* mg = cv.take<uint8_t>(tot.max_mask);
    uint8_t* flag = cv.take<uint8_t>(N);
    int32_t* part = cv.take<int32_t>((size_t)column_order_slices(N) * N);
    double* Jd = cv.take<double>(tot.n_J);
    if (!cv.ok) return fail(VQ_ERR_WORKSPACE, "vq_fit_grouped: workspace too small");
    void* sws = cv.base + cv.used;
    const size_t sws_bytes = cv.cap - cv.used;

    VQ_TRY(select_launch(in->W, in->h, M, N, f.d, nnz, out->row_ptr, out->col, out->val, out->mask, sws, sws_bytes,
                         st));
    const float* X = in->W;
    const float* hc = in->h;
    if (f.binorm) {
        VQ_TRY(binorm_launch(in->W, in->h, M, N, Wp, r, c, hcol, rho, sws, sws_bytes, st));
        X = Wp;
        hc = hcol;
    }
    {
        TimedRegion tr("column_order", 0, st);
        VQ_TRY(column_order_launch(in->h, N, p->n_out, out->cols, flag, part, st));
    }

    int64_t oi = 0, oc = 0, oj = 0, op1 = 0, op2 = 0;
    for (const GroupSpec& g : groups) {
        const int32_t* gc = out->cols + g.c0;
        const int64_t ns = M * g.Ng / g.d;
        const uint8_t* mk = nullptr;
        {
            TimedRegion tr("group_gather", g.K, st);
            VQ_TRY(gather_cols_launch(X, M, N, gc, g.Ng, Xg, st));
            VQ_TRY(gather_cols_launch(hc, 1, N, gc, g.Ng, hg, st));
            if (f.binorm) VQ_TRY(gather_cols_launch(c, 1, N, gc, g.Ng, cg, st));
            if (f.mask_outliers) {
                VQ_TRY(gather_mask_launch(out->mask, M, N, f.d, gc, g.Ng, g.d, mg, st));
                mk = mg;
            }
        }
        uint16_t* i1 = out->idx + oi;
        float* C1 = out->codebooks + oc;
        VQ_TRY(init_walk(Xg, ns, g.d, in->perm1 + op1, g.K, C1, sws, sws_bytes, st));
        VQ_TRY(lloyd_stage(Xg, hg, f.binorm ? rho : nullptr, mk, M, g.Ng, g.d, C1, g.K, g.T, i1, Jd + oj, sws,
                           sws_bytes, st));
        oi += ns; oc += (int64_t)g.K * g.d; oj += g.T + 1; op1 += ns;
        uint16_t* i2 = nullptr;
        float* C2 = nullptr;
        if (g.K2 > 0) {
            i2 = out->idx + oi;
            C2 = out->codebooks + oc;
            VQ_TRY(residual_launch(Xg, M, g.Ng, g.d, C1, g.K, i1, Rg, st));
            VQ_TRY(init_walk(Rg, ns, g.d, in->perm2 + op2, g.K2, C2, sws, sws_bytes, st));
            VQ_TRY(lloyd_stage(Rg, hg, f.binorm ? rho : nullptr, mk, M, g.Ng, g.d, C2, g.K2, g.T2, i2, Jd + oj, sws,
                               sws_bytes, st));
            oi += ns; oc += (int64_t)g.K2 * g.d; oj += g.T2 + 1; op2 += ns;
        }
        VQ_TRY(reconstruct_launch(M, g.Ng, g.d, C1, g.K, i1, C2, g.K2, i2, f.binorm ? r : nullptr,
                                  f.binorm ? cg : nullptr, nullptr, nullptr, nullptr, Wg, st));
        TimedRegion tr("group_scatter", g.K, st);
        VQ_TRY(scatter_cols_launch(Wg, M, g.Ng, gc, out->W_hat, N, st));
    }
    if (nnz > 0) VQ_TRY(sparse_overwrite_launch(M, N, out->row_ptr, out->col, out->val, out->W_hat, st));
    VQ_HIP(hipMemcpyAsync(out->J_hist, Jd, sizeof(double) * tot.n_J, hipMemcpyDeviceToHost, st));
    VQ_HIP(hipStreamSynchronize(st));
    if (out->bpw) *out->bpw = vq_bits_per_weight_grouped(p);
    return VQ_OK;
}

int vq_assign_exact_count(void* ws, size_t ws_bytes, int64_t n_sub, int K, void* stream)
{
    int n = -1;
    if (assign_flag_count(ws, ws_bytes, n_sub, K, &n, as_stream(stream)) != VQ_OK) return -1;
    return n;
}

int64_t vq_assign_exact_list(void* ws, size_t ws_bytes, int64_t n_sub, int K, int32_t* list, int64_t cap,
                             void* stream)
{
    if (!ws || n_sub <= 0 || K < 1 || K > 65536 || cap < 0 || (cap > 0 && !list)) {
        set_error("vq_assign_exact_list: bad argument");
        return -1;
    }
    if (ws_bytes < ws_assign(n_sub, K)) {
        set_error("vq_assign_exact_list: workspace too small");
        return -1;
    }
    int64_t n = -1;
    if (assign_flag_list(ws, ws_bytes, n_sub, K, list, cap, &n, as_stream(stream)) != VQ_OK) return -1;
    return n;
}

int64_t vq_nnz(int64_t M, int64_t N, double p)
{
    if (M <= 0 || N <= 0 || !(p >= 0.0 && p <= 1.0)) {
        set_error("vq_nnz: M, N must be positive and p in [0, 1]");
        return -1;
    }
    return nnz_of(M, N, p);
}

}  // extern "C"
