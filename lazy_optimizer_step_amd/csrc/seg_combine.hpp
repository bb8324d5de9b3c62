// seg_combine.hpp - the segment tiles of the lookup canonicalisation and the
// combine of the sums of segments that cross them, shared by canon.hip (the
// canonicalisation calls) and update.hip (the step from raw lookups, which
// combines a crossing segment and updates its row in one block).
#pragma once

#include "common.hpp"

namespace spopt {

constexpr int kSumWaves = 16;                   // waves per segment-and-sum block
constexpr int kSumThreads = kSumWaves * kWave;
constexpr int kSumRows = 16;                    // sorted lookups per wave (lanes 0..15)
constexpr int kSumTile = kSumWaves * kSumRows;  // sorted lookups per such block
constexpr int kTilePartials = 8;                // partials one wave adds alone in the combine
constexpr int kFixRuns = 16;                    // runs of a segment with more partials

template <int V>
__device__ __forceinline__ void store_row(float* dst, const double (&r)[V], int64_t col,
                                          int64_t width) {
    if (col < width) {
        if constexpr (V == 4) {
            *reinterpret_cast<float4*>(dst) =
                make_float4((float)r[0], (float)r[1], (float)r[2], (float)r[3]);
        } else if constexpr (V == 2) {
            *reinterpret_cast<float2*>(dst) = make_float2((float)r[0], (float)r[1]);
        } else {
            dst[0] = (float)r[0];
        }
    }
}

// Partial sums of segments that cross a chunk boundary stay in double.
template <int V>
__device__ __forceinline__ void load_part(double (&r)[V], const double* src, int64_t col,
                                          int64_t width) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const bool in = col + v < width;
        const double x = src[in ? v : -col];  // past the row: its first column
        r[v] = in ? x : 0.0;
    }
}

// Adds partials q in [lo, hi) of a segment whose start tile is `tile` (q = 0:
// tlast[tile], q > 0: tfirst[tile + q]) in increasing q, D loads in flight
// (past hi, partial lo is reloaded and unused).
template <int V, int D>
__device__ __forceinline__ void add_partials(double (&acc)[V], const double* tfirst,
                                             const double* tlast, int64_t tile, int64_t lo,
                                             int64_t hi, int64_t width, int64_t col) {
    for (int64_t q0 = lo; q0 < hi; q0 += D) {
        double row[D][V];
#pragma unroll
        for (int u = 0; u < D; ++u) {
            const int64_t q = q0 + u < hi ? q0 + u : lo;
            const double* src = (q == 0) ? tlast + tile * width : tfirst + (tile + q) * width;
            load_part<V>(row[u], src + col, col, width);
        }
#pragma unroll
        for (int u = 0; u < D; ++u)
            if (q0 + u < hi) {
#pragma unroll
                for (int v = 0; v < V; ++v) acc[v] += row[u][v];
            }
    }
}

// Segments that cross tiles, one block per tile that starts one (tcross):
// m partials (tlast of the start tile, tfirst of each following tile up to
// the one where it ends).  The order of the additions depends on m only, so
// the result is the same run to run and whatever the block's shape: up to
// kTilePartials partials are added in tile order by wave 0; beyond, [0, m) is
// cut into kFixRuns equal runs, each added in tile order (run r by wave
// r mod W), and wave 0 adds the run sums in run order.  The block also writes
// the segment's count.  part: LDS, kFixRuns rows.  Returns the segment (the
// same value in every thread), or -1 when the tile starts none or the status
// word holds an error.
template <int V, int W>
__device__ __forceinline__ int32_t tile_fixup_body(
    int64_t tile, const int32_t* __restrict__ tcross, const int32_t* __restrict__ seg_start,
    const double* __restrict__ tfirst, const double* __restrict__ tlast, int64_t width,
    float* __restrict__ out_vals, int32_t* __restrict__ out_counts, const uint32_t* status,
    double (*part)[kWave * V]) {
    const uint32_t st0 = *status;  // loaded together with the crossing segment
    const int32_t seg = tcross[tile];
    if (st0 != 0u || seg < 0) return -1;
    const int w = (int)(threadIdx.x >> 6);
    const int lane = lane_id();
    const int64_t s0 = seg_start[seg], s1 = seg_start[seg + 1];
    if (threadIdx.x == 0) out_counts[seg] = (int32_t)(s1 - s0);
    const int64_t m = (s1 - 1) / kSumTile - tile + 1;
    for (int64_t c0 = 0; c0 < width; c0 += (int64_t)kWave * V) {
        const int64_t col = c0 + (int64_t)lane * V;
        if (m <= kTilePartials) {
            if (w == 0) {
                double tot[V];
#pragma unroll
                for (int v = 0; v < V; ++v) tot[v] = 0.0;
                add_partials<V, (V == 4 ? 4 : 8)>(tot, tfirst, tlast, tile, 0, m, width, col);
                store_row<V>(out_vals + (int64_t)seg * width + col, tot, col, width);
            }
            continue;
        }
        for (int r = w; r < kFixRuns; r += W) {
            const int64_t lo = m * r / kFixRuns, hi = m * (r + 1) / kFixRuns;
            double acc[V];
#pragma unroll
            for (int v = 0; v < V; ++v) acc[v] = 0.0;
            add_partials<V, (V == 4 ? 4 : 8)>(acc, tfirst, tlast, tile, lo, hi, width, col);
#pragma unroll
            for (int v = 0; v < V; ++v) part[r][lane * V + v] = acc[v];
        }
        __syncthreads();
        if (w == 0) {
            double tot[V];
#pragma unroll
            for (int v = 0; v < V; ++v) tot[v] = part[0][lane * V + v];
            for (int r = 1; r < kFixRuns; ++r)
#pragma unroll
                for (int v = 0; v < V; ++v) tot[v] += part[r][lane * V + v];
            store_row<V>(out_vals + (int64_t)seg * width + col, tot, col, width);
        }
        __syncthreads();
    }
    return seg;
}

}  // namespace spopt
