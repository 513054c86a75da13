// Internal helpers of libvq: status/error plumbing, workspace carving and
// small device utilities shared by the kernel files.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/vq.h"

namespace vq {

// ---- errors -------------------------------------------------------------
void set_error(const std::string& msg);
vq_status fail(vq_status st, const std::string& msg);
vq_status hip_fail(hipError_t e, const char* what);

#define VQ_HIP(call)                                              \
    do {                                                          \
        hipError_t vq_e_ = (call);                                \
        if (vq_e_ != hipSuccess) return ::vq::hip_fail(vq_e_, #call); \
    } while (0)

#define VQ_CHECK(cond, msg)                                       \
    do {                                                          \
        if (!(cond)) return ::vq::fail(VQ_ERR_INVALID, (msg));    \
    } while (0)

#define VQ_LAUNCHED(name)                                         \
    do {                                                          \
        hipError_t vq_e_ = hipGetLastError();                     \
        if (vq_e_ != hipSuccess) return ::vq::hip_fail(vq_e_, name); \
    } while (0)

// ---- workspace ----------------------------------------------------------
constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Hands out aligned slices of the caller's workspace in order.
struct Carver {
    char* base;
    size_t cap;
    size_t used = 0;
    bool ok = true;
    Carver(void* p, size_t bytes) : base(static_cast<char*>(p)), cap(bytes) {}
    template <class T>
    T* take(size_t count) {
        size_t b = align_up(count * sizeof(T));
        if (used + b > cap || base == nullptr) { ok = false; return nullptr; }
        T* p = reinterpret_cast<T*>(base + used);
        used += b;
        return p;
    }
};

// Workspace needs of each step (bytes); must match the carving in each file.
size_t ws_assign(int64_t n_sub, int K);
size_t ws_assign_full(int64_t n_sub, int K);
size_t ws_update(int64_t n_sub, int K);
size_t ws_objective(int64_t n_sub);
size_t ws_select(int64_t M, int64_t N);
size_t ws_binorm(int64_t M, int64_t N);
size_t ws_init(int64_t n_sub, int K, int d);
size_t ws_qgemv(int64_t M, int64_t N, int d, int64_t B);
size_t ws_vptq(int64_t M, int64_t N, int V);
size_t ws_hfactor(int64_t N);

// Argument checks shared by the entry points.
vq_status check_shape(int64_t M, int64_t N, int d);
vq_status check_K(int K, int64_t n_sub);

// Input value checks (environment VQ_CHECK=1): counts the non-finite values of
// a[0..n) (with sign_clear, also those with the sign bit set) on the device and
// fails with VQ_ERR_INVALID naming `what` if any.  A no-op when the mode is off
// or a is null.  Synchronizes st when on.
bool values_check_on();
vq_status check_values(const float* a, int64_t n, bool sign_clear, const char* call, const char* what,
                       hipStream_t st);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Brackets the launches in its scope with events on `st` when timing is on
// (vq_timing_enable); a no-op otherwise.
class TimedRegion {
  public:
    TimedRegion(const char* name, int K, hipStream_t st);
    ~TimedRegion();
    TimedRegion(const TimedRegion&) = delete;
    TimedRegion& operator=(const TimedRegion&) = delete;

  private:
    const char* name_;
    int K_;
    hipStream_t st_;
    void* a_ = nullptr;
};

// Diagnostics beside the timing records: whether timing is on, and a count
// added to the launches of record (name, K) (no time) while it is.
bool timing_on();
void timing_count(const char* name, int K, int64_t n);

inline unsigned grid_for(int64_t work, int per_block) {
    int64_t g = (work + per_block - 1) / per_block;
    return static_cast<unsigned>(g < 1 ? 1 : g);
}

}  // namespace vq
