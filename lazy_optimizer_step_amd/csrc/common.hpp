// common.hpp - device helpers and host plumbing shared by the HIP sources of
// the sparse / lazy optimizer library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "sparse_opt.h"

namespace spopt {

constexpr int kWave = 64;

// Device-side status bits, OR-ed into a status word by checking kernels.
enum : uint32_t {
    kStatusRange = 1u,     // index outside its range
    kStatusNotCanon = 2u,  // not strictly ascending / CSR not canonical
    kStatusNonFinite = 4u, // NaN or inf gradient value
    kStatusStep = 8u,      // last_step >= t on a touched coordinate
    kStatusTouched = 16u,  // touched-row list inconsistent with row_offsets
    kStatusTimeout = 32u,  // a bounded device-side wait gave up (a library bug)
    kStatusPartial = 64u   // a partial row given to a table with one last_step per row
};

// ---------------------------------------------------------------- device ---

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ __forceinline__ uint64_t ballot(bool p) { return (uint64_t)__ballot(p); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int l = lane_id();
    return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ int popc64(uint64_t x) { return __popcll(x); }

template <class T>
__device__ __forceinline__ T read_lane(T v, int lane);

template <>
__device__ __forceinline__ int read_lane<int>(int v, int lane) {
    return __builtin_amdgcn_readlane(v, lane);
}
template <>
__device__ __forceinline__ uint32_t read_lane<uint32_t>(uint32_t v, int lane) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
    const int l = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        uint32_t y = __shfl_up(x, off, kWave);
        if (l >= off) x += y;
    }
    return x;
}

// Exclusive prefix sum over a block; `warp_tot` is LDS scratch with one slot
// per wave of the block.  Returns the exclusive prefix; *total gets the sum.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t x, uint32_t* warp_tot,
                                                    uint32_t* total) {
    const int w = (int)(threadIdx.x >> 6);
    const int nw = (int)((blockDim.x + kWave - 1) >> 6);
    uint32_t inc = wave_incl_scan(x);
    if (lane_id() == kWave - 1) warp_tot[w] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
    for (int i = 0; i < nw; ++i) {
        uint32_t t = warp_tot[i];
        if (i < w) before += t;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + inc - x;
}

__device__ __forceinline__ bool finite_f(float x) { return __builtin_isfinite(x); }

// Division of unsigned 64-bit integers by a divisor fixed for a launch,
// without the GPU's long software division: with s = floor(log2 d) and
// m = floor((2^(64+s) - 1) / d), formed on the host, the estimate
// q = high64(n * m) >> s falls short of floor(n / d) by at most 1 for every
// n < 2^64 (m * 2^-(64+s) undershoots 1/d by less than 2^-(64+s)), so one
// correction step gives the exact quotient.
struct FastDiv {
    uint64_t d, m;
    int s;
    static FastDiv make(uint64_t d) {
        FastDiv f;
        f.d = d;
        f.s = 63 - __builtin_clzll(d);
        f.m = (uint64_t)((((unsigned __int128)1 << (64 + f.s)) - 1) / d);
        return f;
    }
    __device__ __forceinline__ uint64_t div(uint64_t n, uint64_t* rem = nullptr) const {
        uint64_t q = __umul64hi(n, m) >> s;
        uint64_t r = n - q * d;
        if (r >= d) {
            ++q;
            r -= d;
        }
        if (rem) *rem = r;
        return q;
    }
};

// ------------------------------------------------------------------ host ---

void set_error(const char* fmt, ...);
int fail(int code, const char* fmt, ...);

#define SPOPT_HIP(call)                                                                   \
    do {                                                                                  \
        hipError_t e_ = (call);                                                           \
        if (e_ != hipSuccess)                                                             \
            return ::spopt::fail(SPOPT_EDEVICE, "%s failed: %s", #call,                   \
                                 hipGetErrorString(e_));                                  \
    } while (0)

#define SPOPT_LAUNCHED()                                                                  \
    do {                                                                                  \
        hipError_t e_ = hipGetLastError();                                                \
        if (e_ != hipSuccess)                                                             \
            return ::spopt::fail(SPOPT_EDEVICE, "kernel launch failed: %s",               \
                                 hipGetErrorString(e_));                                  \
    } while (0)

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

__host__ __device__ inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Status-word helpers implemented in abi.hip.
int status_to_code(uint32_t bits, const char* what);
std::mutex& validation_mutex();
uint32_t* device_status_block();  // 4 words per device, allocated on first use
int device_status_check(uint32_t* d_status, hipStream_t s, bool check_touched,
                        const char* what);

// Launchers shared between the sources.
int launch_status_clear(uint32_t* d_status, int nwords, hipStream_t s);
// last_step of the coordinate (row, col) is ls[row * ls_rs + col * ls_cs]:
// (cols, 1) per coordinate, (1, 0) per row.  full_rows: a row with some but
// not all of its columns sets kStatusPartial.
struct LastStepView {
    const int32_t* ls;
    int32_t t;
    int64_t ls_rs, ls_cs;
    int full_rows;
};

int launch_check_coo(const spopt_coo* c, int check_finite, const LastStepView& lv,
                     uint32_t* status, hipStream_t s);
int launch_check_csr(const spopt_csr* c, int check_finite, const LastStepView& lv,
                     uint32_t* status, hipStream_t s);

// beta^gap for gap < kPowTable comes from a table built on the host with pow().
constexpr int kPowTable = 1024;

// Per-step scalars of Adam, formed in double on the host.
// Weight decay of an Adam step: none (weight_decay == 0), into the gradient,
// or beside the move.
enum : int { kWdNone = 0, kWdL2 = 1, kWdDecoupled = 2 };

struct AdamScalars {
    double lr, c1, c2, bc1, bc2, eps, beta1, beta2, l2b1, l2b2;
    double wd, lr_wd;    // weight_decay and lr * weight_decay
    const double* pow1;  // device [kPowTable]: beta1^k
    const double* pow2;  // device [kPowTable]: beta2^k
    int32_t t;
};
// The calling thread's timing events (sparse_opt_set_step_events), both NULL
// when none are set: attached to the dispatch of every kernel that updates a
// table, they take its start and end times.
struct StepEvents {
    hipEvent_t begin, end;
};
StepEvents step_events();

int launch_adam(float* p, float* m, float* v, int32_t* ls, bool ls_per_row, const AdamScalars& a,
                int mode, int wd_kind, const spopt_grad* gr, int64_t rows, int64_t cols,
                hipStream_t s);
int launch_sgd(float* p, float* b, double lr, double mu, double wd, const spopt_grad* gr,
               int64_t rows, int64_t cols, hipStream_t s);

// What is left of csr_from_lookups after its segment kernel, when a step from
// raw lookups finishes it in the update's own launch: the combine of the
// segments that cross segment tiles (nfix blocks, one per tile), the
// col_indices blocks (nblk_ci, none without col_indices) and the row_offsets
// blocks (nblk_ro).  keys/vals/counts are the canonical outputs (n lookups at
// most; the distinct count on the device at d_n); tcross .. status point into
// the call's workspace; bnd (or NULL) holds the id counts below each 8192-row
// block.  row_offsets is 16-byte aligned and cols a multiple of 4.
struct FusedCsr {
    const int32_t* tcross;
    const int32_t* seg_start;
    const double* tfirst;
    const double* tlast;
    const uint32_t* status;
    int64_t nfix;
    const int64_t* keys;
    float* vals;
    int32_t* counts;
    const int64_t* d_n;
    int64_t n, rows, cols;
    int32_t* row_offsets;
    int32_t* col_indices;
    const int32_t* bnd;
    int64_t nblk_ci, nblk_ro;
};

// csr_from_lookups with `defer` != NULL: when the call can hand its last
// launch over (trusted, cols % 4 == 0, row_offsets and col_indices 16-byte
// aligned) it fills *defer and returns with *deferred = true; otherwise it
// completes the CSR itself (*deferred = false).  `what` names the entry
// point in errors.
int csr_lookups_run(const char* what, const int64_t* ids, const float* vals, int64_t n,
                    int64_t rows, int64_t cols, int64_t* out_keys, float* out_vals,
                    int32_t* out_counts, int64_t* d_nunique, int32_t* row_offsets,
                    int32_t* col_indices, void* workspace, size_t workspace_bytes, hipStream_t s,
                    uint32_t flags, FusedCsr* defer, bool* deferred);
int launch_adam_fused(float* p, float* m, float* v, int32_t* ls, bool ls_per_row,
                      const AdamScalars& a, int mode, int wd_kind, const FusedCsr& f,
                      hipStream_t s);
int launch_sgd_fused(float* p, float* b, double lr, double mu, double wd, const FusedCsr& f,
                     hipStream_t s);

// A validated call: serialised with every other validated call of the
// process, it clears the device's status block, lets `launch` enqueue its
// checks into it, and reads it back (one synchronisation of `s`).
template <class F>
int validate_on_device(hipStream_t s, bool check_touched, const char* what, F&& launch) {
    std::lock_guard<std::mutex> guard(validation_mutex());
    uint32_t* status = device_status_block();
    if (status == nullptr) return fail(SPOPT_EDEVICE, "%s: no device status block", what);
    int rc = launch_status_clear(status, 4, s);
    if (rc) return rc;
    rc = launch(status);
    if (rc) return rc;
    return device_status_check(status, s, check_touched, what);
}

}  // namespace spopt
