// rows.hip - forward gather of table rows (read_rows).
//
// DiskSparseAdam README, API reference, read_rows(indices): the rows of the
// current table for a batch of lookup indices, duplicates allowed, indices
// validated, corrupted rows refused.  On the GPU the table's pending writes are
// the update kernels earlier on the same stream, so stream order gives the
// read-after-write the README obtains by draining its writer.  The hyperbolic
// projection of that page is outside the Euclidean method built here.
#include "common.hpp"

namespace spopt {

constexpr int kGatherRows = 16;  // rows per wave, all loads in flight together

// One wave per kGatherRows lookups; LPR lanes x V floats cover LPR*V
// consecutive columns of one row, so one load instruction moves 64/LPR rows.
// For each block of columns every row is loaded first (straight-line: an
// index outside the table loads row 0 and stores zeros), then stored.
template <int V, int LPR>
__global__ __launch_bounds__(256) void k_read_rows(const float* __restrict__ params, int64_t rows,
                                                   int64_t cols, const int64_t* __restrict__ idx,
                                                   int64_t n, float* __restrict__ out) {
    constexpr int RPI = kWave / LPR;
    constexpr int U = kGatherRows / RPI;
    const int lane = lane_id();
    const int sub = lane / LPR, sl = lane % LPR;
    const int64_t k0 = (((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6) * kGatherRows;
    if (k0 >= n) return;
    int64_t src[U];
    bool ok[U], live[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t k = k0 + u * RPI + sub;
        live[u] = k < n;
        const int64_t r = idx[live[u] ? k : k0];
        ok[u] = live[u] && (uint64_t)r < (uint64_t)rows;
        src[u] = ok[u] ? r : 0;
    }
    for (int64_t c0 = 0; c0 < cols; c0 += (int64_t)LPR * V) {
        const int64_t col = c0 + (int64_t)sl * V;
        const bool in = col < cols;
        float x[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float* p = params + src[u] * cols + (in ? col : 0);
            if constexpr (V == 4) {
                const float4 q = *reinterpret_cast<const float4*>(p);
                x[u][0] = q.x; x[u][1] = q.y; x[u][2] = q.z; x[u][3] = q.w;
            } else if constexpr (V == 2) {
                const float2 q = *reinterpret_cast<const float2*>(p);
                x[u][0] = q.x; x[u][1] = q.y;
            } else {
                x[u][0] = p[0];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (!live[u] || !in) continue;
            const int64_t k = k0 + u * RPI + sub;
            float* o = out + k * cols + col;
            if constexpr (V == 4) {
                *reinterpret_cast<float4*>(o) = ok[u] ? make_float4(x[u][0], x[u][1], x[u][2], x[u][3])
                                                      : make_float4(0.f, 0.f, 0.f, 0.f);
            } else if constexpr (V == 2) {
                *reinterpret_cast<float2*>(o) = ok[u] ? make_float2(x[u][0], x[u][1])
                                                      : make_float2(0.f, 0.f);
            } else {
                o[0] = ok[u] ? x[u][0] : 0.f;
            }
        }
    }
}

// Validation: every index in range and every gathered value finite (one wave
// per lookup row).
__global__ void k_check_rows(const float* __restrict__ params, int64_t rows, int64_t cols,
                             const int64_t* __restrict__ idx, int64_t n, uint32_t* status) {
    const int lane = lane_id();
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    uint32_t bad = 0;
    for (int64_t k = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6; k < n; k += nw) {
        const int64_t r = idx[k];
        if ((uint64_t)r >= (uint64_t)rows) {
            bad |= kStatusRange;
            continue;
        }
        for (int64_t c = lane; c < cols; c += kWave)
            if (!finite_f(params[r * cols + c])) bad |= kStatusNonFinite;
    }
    if (bad) atomicOr(status, bad);
}

}  // namespace spopt

using namespace spopt;

extern "C" int read_rows(const float* params, int64_t rows, int64_t cols, const int64_t* indices,
                         int64_t n, float* out, void* stream, uint32_t flags) {
    hipStream_t st = (hipStream_t)stream;
    if (params == nullptr || rows < 1 || cols < 1 || n < 0)
        return fail(SPOPT_EINVAL, "read_rows: NULL table or bad size");
    if (n > 0 && (indices == nullptr || out == nullptr))
        return fail(SPOPT_EINVAL, "read_rows: NULL indices or output");
    if (n == 0) return SPOPT_OK;
    if (flags & SPOPT_VALIDATE) {
        const int rc = validate_on_device(st, false, "read_rows", [&](uint32_t* status) -> int {
            const int64_t g = ceil_div(n, 4);
            k_check_rows<<<(unsigned)(g < 4096 ? g : 4096), 256, 0, st>>>(params, rows, cols,
                                                                        indices, n, status);
            SPOPT_LAUNCHED();
            return SPOPT_OK;
        });
        if (rc) return rc;
    }
    const uintptr_t al = (uintptr_t)params | (uintptr_t)out;
    const int V = (cols % 4 == 0 && (al & 15u) == 0) ? 4 : (cols % 2 == 0 && (al & 7u) == 0) ? 2 : 1;
    const int lpr = cols <= 16 * V ? 16 : (cols <= 32 * V ? 32 : 64);
    const unsigned grid = (unsigned)ceil_div(ceil_div(n, kGatherRows), 4);
    auto go = [&](auto kernel) {
        kernel<<<grid, 256, 0, st>>>(params, rows, cols, indices, n, out);
    };
    if (V == 4)
        lpr == 16 ? go(k_read_rows<4, 16>) : lpr == 32 ? go(k_read_rows<4, 32>)
                                                      : go(k_read_rows<4, 64>);
    else if (V == 2)
        lpr == 16 ? go(k_read_rows<2, 16>) : lpr == 32 ? go(k_read_rows<2, 32>)
                                                      : go(k_read_rows<2, 64>);
    else
        lpr == 16 ? go(k_read_rows<1, 16>) : lpr == 32 ? go(k_read_rows<1, 32>)
                                                      : go(k_read_rows<1, 64>);
    SPOPT_LAUNCHED();
    return SPOPT_OK;
}
