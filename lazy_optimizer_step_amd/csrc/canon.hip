// canon.hip - raw lookups -> canonical COO on the GPU.
//
// Computes what the DiskSparseAdam README calls "Safe Duplicate Aggregation &
// Sorted I/O" (duplicates summed, indices sorted) and what the optirs_gpu
// sparse_optimizer page requires of a CooGradient (strictly ascending
// indices):
//   1. pack each lookup as (id << pos_bits) | position and radix-sort the
//      packed words on the id bits only (LSD, 8-bit digits, stable, so equal
//      ids keep lookup order);
//   2. mark segment heads (id differs from its predecessor), scan them to give
//      every lookup its segment number and emit the distinct ids;
//   3. sum each segment's value rows in double, in a fixed order, and round
//      once: fixed chunks of 64 sorted lookups per wave, partial sums for
//      segments that cross a chunk boundary, then an ordered combine of those
//      partials.  No atomics, so the result is the same run to run.
#include <stdarg.h>
#include <stdio.h>

#include "common.hpp"

namespace spopt {

constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / kWave;
constexpr int kSortIpt = 4;                                  // items per thread
constexpr int kSortTile = kSortThreads * kSortIpt;           // 1024 lookups per block
constexpr int kRadixBits = 8;
constexpr int kRadix = 1 << kRadixBits;
constexpr int kSegTile = 1024;                                // lookups per block, segmenting
constexpr int kChunk = 64;                                    // lookups per wave, summing

struct CanonLayout {
    int key_bits, pos_bits, passes;
    int64_t nblk_sort, nblk_seg, nchunks;
    size_t off_a, off_b, off_hist, off_blk, off_segid, off_segstart, off_pfirst, off_plast,
        off_status, total;
};

static int bits_for(uint64_t x) {  // bits needed to represent values in [0, x)
    int b = 0;
    while (b < 64 && (x - 1) >> b) ++b;
    return x <= 1 ? 0 : b;
}

static bool canon_layout(int64_t n, int64_t width, int64_t key_space, CanonLayout* L) {
    if (n < 0 || width < 1 || key_space < 1) return false;
    L->key_bits = bits_for((uint64_t)key_space);
    L->pos_bits = bits_for((uint64_t)(n > 0 ? n : 1));
    if (L->key_bits + L->pos_bits > 64) return false;
    L->passes = (L->key_bits + kRadixBits - 1) / kRadixBits;
    L->nblk_sort = ceil_div(n, kSortTile);
    L->nblk_seg = ceil_div(n, kSegTile);
    L->nchunks = ceil_div(n, kChunk);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes, 256);
        return at;
    };
    L->off_a = take(sizeof(uint64_t) * (size_t)n);
    L->off_b = take(sizeof(uint64_t) * (size_t)n);
    L->off_hist = take(sizeof(uint32_t) * (size_t)kRadix * (size_t)L->nblk_sort);
    L->off_blk = take(sizeof(uint32_t) * ((size_t)L->nblk_seg + 1));
    L->off_segid = take(sizeof(int32_t) * (size_t)n);
    L->off_segstart = take(sizeof(int32_t) * ((size_t)n + 1));
    L->off_pfirst = take(sizeof(double) * (size_t)L->nchunks * (size_t)width);
    L->off_plast = take(sizeof(double) * (size_t)L->nchunks * (size_t)width);
    L->off_status = take(sizeof(uint32_t) * 4);
    L->total = o;
    return true;
}

// ------------------------------------------------------------------ sort ---

__global__ void k_status_clear(uint32_t* st, int nwords) {
    if ((int)threadIdx.x < nwords) st[threadIdx.x] = 0u;
}

// Pass 0: range-check ids, pack (id, position), digit histogram of this block.
__global__ __launch_bounds__(kSortThreads) void k_pack_hist(
    const int64_t* __restrict__ ids, int64_t n, int64_t key_space, int pos_bits, int shift,
    uint32_t mask, uint64_t* __restrict__ out, uint32_t* __restrict__ hist, int64_t nblk,
    int do_hist, uint32_t* status) {
    __shared__ uint32_t h[kRadix];
    for (int i = threadIdx.x; i < kRadix; i += blockDim.x) h[i] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kSortTile;
    bool bad = false;
#pragma unroll
    for (int j = 0; j < kSortIpt; ++j) {
        const int64_t i = base + (int64_t)j * kSortThreads + threadIdx.x;
        if (i < n) {
            int64_t id = ids[i];
            if (id < 0 || id >= key_space) {
                bad = true;
                id = 0;  // keep sorting a safe key; the result is discarded
            }
            const uint64_t packed = ((uint64_t)id << pos_bits) | (uint64_t)i;
            out[i] = packed;
            if (do_hist) atomicAdd(&h[(uint32_t)(packed >> shift) & mask], 1u);
        }
    }
    if (ballot(bad) != 0ull && lane_id() == 0) atomicOr(status, kStatusRange);
    if (!do_hist) return;
    __syncthreads();
    for (int d = threadIdx.x; d < kRadix; d += blockDim.x) hist[(int64_t)d * nblk + blockIdx.x] = h[d];
}

// Digit histogram of one block for passes after the first.
__global__ __launch_bounds__(kSortThreads) void k_hist(const uint64_t* __restrict__ in, int64_t n,
                                                       int shift, uint32_t mask,
                                                       uint32_t* __restrict__ hist, int64_t nblk) {
    __shared__ uint32_t h[kRadix];
    for (int i = threadIdx.x; i < kRadix; i += blockDim.x) h[i] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kSortTile;
#pragma unroll
    for (int j = 0; j < kSortIpt; ++j) {
        const int64_t i = base + (int64_t)j * kSortThreads + threadIdx.x;
        if (i < n) atomicAdd(&h[(uint32_t)(in[i] >> shift) & mask], 1u);
    }
    __syncthreads();
    for (int d = threadIdx.x; d < kRadix; d += blockDim.x) hist[(int64_t)d * nblk + blockIdx.x] = h[d];
}

// In-place exclusive scan of a uint32 array by one block of 1024 threads; each
// thread owns one contiguous segment.
__global__ __launch_bounds__(1024) void k_scan_u32(uint32_t* data, int64_t len) {
    __shared__ uint32_t wt[16];
    const int64_t per = (len + blockDim.x - 1) / blockDim.x;
    const int64_t beg = (int64_t)threadIdx.x * per;
    const int64_t end = beg + per < len ? beg + per : len;
    uint32_t sum = 0;
    for (int64_t i = beg; i < end; ++i) sum += data[i];
    uint32_t total;
    uint32_t off = block_excl_scan(sum, wt, &total);
    for (int64_t i = beg; i < end; ++i) {
        uint32_t x = data[i];
        data[i] = off;
        off += x;
    }
}

// Stable scatter of one radix pass.  Wave w of a block ranks the block's items
// [w*256, (w+1)*256) in four rounds of 64 consecutive items: lanes holding the
// same digit are found with 8 ballots, each lane's rank is the number of
// lower lanes with its digit plus the wave's running count of that digit.
__global__ __launch_bounds__(kSortThreads) void k_scatter(const uint64_t* __restrict__ in,
                                                          uint64_t* __restrict__ out, int64_t n,
                                                          int shift, uint32_t mask, int nbits,
                                                          const uint32_t* __restrict__ hist,
                                                          int64_t nblk) {
    __shared__ uint32_t cnt[kSortWaves][kRadix];
    const int w = (int)(threadIdx.x >> 6);
    const int lane = lane_id();
    for (int i = threadIdx.x; i < kSortWaves * kRadix; i += blockDim.x) (&cnt[0][0])[i] = 0;
    __syncthreads();

    const int64_t base = (int64_t)blockIdx.x * kSortTile + (int64_t)w * (kSortIpt * kWave);
    const uint64_t lt = lanemask_lt();
    uint64_t key[kSortIpt];
    uint32_t dig[kSortIpt], rank[kSortIpt];
    bool valid[kSortIpt];
#pragma unroll
    for (int r = 0; r < kSortIpt; ++r) {
        const int64_t i = base + (int64_t)r * kWave + lane;
        valid[r] = i < n;
        key[r] = valid[r] ? in[i] : 0ull;
        dig[r] = (uint32_t)(key[r] >> shift) & mask;
    }
#pragma unroll
    for (int r = 0; r < kSortIpt; ++r) {
        uint64_t peers = ballot(valid[r]);
        for (int b = 0; b < nbits; ++b) {
            const bool bit = (dig[r] >> b) & 1u;
            const uint64_t bb = ballot(bit);
            peers &= bit ? bb : ~bb;
        }
        const uint32_t below = (uint32_t)popc64(peers & lt);
        uint32_t old = 0;
        if (valid[r]) old = cnt[w][dig[r]];
        // Every lane of the wave reads the counter in the same LDS instruction,
        // before the group's lowest lane writes the new count (its store
        // depends on the value read, and one wave's LDS operations complete in
        // program order).
        if (valid[r] && below == 0) cnt[w][dig[r]] = old + (uint32_t)popc64(peers);
        rank[r] = old + below;
    }
    __syncthreads();
    for (int d = threadIdx.x; d < kRadix; d += blockDim.x) {
        uint32_t run = hist[(int64_t)d * nblk + blockIdx.x];
        for (int ww = 0; ww < kSortWaves; ++ww) {
            const uint32_t c = cnt[ww][d];
            cnt[ww][d] = run;
            run += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSortIpt; ++r)
        if (valid[r]) out[cnt[w][dig[r]] + rank[r]] = key[r];
}

// ------------------------------------------------------------- segments ---

__device__ __forceinline__ bool seg_head(const uint64_t* s, int64_t i, int pos_bits) {
    return i == 0 || (s[i] >> pos_bits) != (s[i - 1] >> pos_bits);
}

__global__ __launch_bounds__(256) void k_seg_count(const uint64_t* __restrict__ s, int64_t n,
                                                   int pos_bits, uint32_t* __restrict__ blk) {
    __shared__ uint32_t wt[4];
    const int64_t base = (int64_t)blockIdx.x * kSegTile;
    uint32_t c = 0;
    for (int j = 0; j < kSegTile / 256; ++j) {
        const int64_t i = base + (int64_t)j * 256 + threadIdx.x;
        if (i < n && seg_head(s, i, pos_bits)) ++c;
    }
    uint32_t total;
    block_excl_scan(c, wt, &total);
    if (threadIdx.x == 0) blk[blockIdx.x] = total;
}

// Scan the per-block head counts; publish U (0 when an id was out of range)
// and the sentinel seg_start[U] = n.
__global__ __launch_bounds__(1024) void k_seg_scan(uint32_t* blk, int64_t nblk, int64_t n,
                                                   int32_t* seg_start, int64_t* d_nunique,
                                                   const uint32_t* status) {
    __shared__ uint32_t wt[16];
    const int64_t per = (nblk + blockDim.x - 1) / blockDim.x;
    const int64_t beg = (int64_t)threadIdx.x * per;
    const int64_t end = beg + per < nblk ? beg + per : nblk;
    uint32_t sum = 0;
    for (int64_t i = beg; i < end; ++i) sum += blk[i];
    uint32_t total;
    uint32_t off = block_excl_scan(sum, wt, &total);
    for (int64_t i = beg; i < end; ++i) {
        uint32_t x = blk[i];
        blk[i] = off;
        off += x;
    }
    if (threadIdx.x == 0) {
        const bool ok = *status == 0u;
        *d_nunique = ok ? (int64_t)total : 0;
        seg_start[total] = (int32_t)n;
    }
}

// Segment number of every sorted lookup; distinct ids and segment starts.
__global__ __launch_bounds__(256) void k_seg_emit(const uint64_t* __restrict__ s, int64_t n,
                                                  int pos_bits, const uint32_t* __restrict__ blk,
                                                  int32_t* __restrict__ seg_id,
                                                  int32_t* __restrict__ seg_start,
                                                  int64_t* __restrict__ out_keys,
                                                  const uint32_t* status) {
    if (*status != 0u) return;
    __shared__ uint32_t wt[4];
    const int64_t base = (int64_t)blockIdx.x * kSegTile;
    uint32_t run = blk[blockIdx.x];
    for (int j = 0; j < kSegTile / 256; ++j) {
        const int64_t i = base + (int64_t)j * 256 + threadIdx.x;
        const bool h = i < n && seg_head(s, i, pos_bits);
        uint32_t total;
        const uint32_t before = block_excl_scan(h ? 1u : 0u, wt, &total);
        if (i < n) {
            const uint32_t seg = run + before + (h ? 1u : 0u) - 1u;
            seg_id[i] = (int32_t)seg;
            if (h) {
                out_keys[seg] = (int64_t)(s[i] >> pos_bits);
                seg_start[seg] = (int32_t)i;
            }
        }
        run += total;
    }
}

// ----------------------------------------------------------- dup sums ---

// V-wide access to a row of floats: a vector load when the layout allows, a
// scalar loop with a column bound otherwise.
template <int V>
__device__ __forceinline__ void load_row(float (&r)[V], const float* src, int64_t col,
                                         int64_t width, bool vec) {
    if (V == 4 && vec && col < width) {
        const float4 x = *reinterpret_cast<const float4*>(src);
        r[0] = x.x; r[1 % V] = x.y; r[2 % V] = x.z; r[3 % V] = x.w;
    } else if (V == 2 && vec && col < width) {
        const float2 x = *reinterpret_cast<const float2*>(src);
        r[0] = x.x; r[1 % V] = x.y;
    } else {
#pragma unroll
        for (int v = 0; v < V; ++v) r[v] = (col + v < width) ? src[v] : 0.f;
    }
}

template <int V>
__device__ __forceinline__ void store_row(float* dst, const double (&r)[V], int64_t col,
                                          int64_t width, bool vec) {
    if (V == 4 && vec && col < width) {
        *reinterpret_cast<float4*>(dst) =
            make_float4((float)r[0], (float)r[1 % V], (float)r[2 % V], (float)r[3 % V]);
    } else if (V == 2 && vec && col < width) {
        *reinterpret_cast<float2*>(dst) = make_float2((float)r[0], (float)r[1 % V]);
    } else {
#pragma unroll
        for (int v = 0; v < V; ++v)
            if (col + v < width) dst[v] = (float)r[v];
    }
}

// Partial sums of segments that cross a chunk boundary stay in double.
template <int V>
__device__ __forceinline__ void load_part(double (&r)[V], const double* src, int64_t col,
                                          int64_t width) {
#pragma unroll
    for (int v = 0; v < V; ++v) r[v] = (col + v < width) ? src[v] : 0.0;
}

template <int V>
__device__ __forceinline__ void store_part(double* dst, const double (&r)[V], int64_t col,
                                           int64_t width) {
#pragma unroll
    for (int v = 0; v < V; ++v)
        if (col + v < width) dst[v] = r[v];
}

// Destination of the running sum when item j of a chunk closes it.
enum : int { kFlushNone = 0, kFlushOut = 1, kFlushFirst = 2, kFlushLast = 3 };

struct ChunkItem {
    uint32_t pos;   // lookup position
    int32_t seg;    // segment number
    int kind;       // kFlush*
    bool ends;      // this lookup is the last of its segment
};

__device__ __forceinline__ ChunkItem chunk_item(const uint64_t* s, const int32_t* seg_id,
                                                const int32_t* seg_start, int64_t n,
                                                int pos_bits, int64_t i0, int cnt, int lane) {
    ChunkItem it{0u, -1, kFlushNone, false};
    if (lane < cnt) {
        const int64_t i = i0 + lane;
        it.pos = (uint32_t)(s[i] & ((pos_bits == 64) ? ~0ull : ((1ull << pos_bits) - 1ull)));
        it.seg = seg_id[i];
        it.ends = (i + 1 >= n) || seg_id[i + 1] != it.seg;
        if (it.ends || lane == cnt - 1) {
            const bool starts_here = seg_start[it.seg] >= i0;
            if (it.ends && starts_here)
                it.kind = kFlushOut;
            else if (!starts_here)
                it.kind = kFlushFirst;
            else
                it.kind = kFlushLast;
        }
    }
    return it;
}

// One wave per chunk of 64 sorted lookups, value rows of `width` floats; each
// lane owns V consecutive columns of every 64*V-column block and accumulates
// them in double, in sorted (= lookup) order within the chunk.
template <int V>
__global__ __launch_bounds__(256) void k_dupsum_rows(
    const uint64_t* __restrict__ s, const int32_t* __restrict__ seg_id,
    const int32_t* __restrict__ seg_start, int64_t n, int pos_bits,
    const float* __restrict__ vals, int64_t width, float* __restrict__ out_vals,
    int32_t* __restrict__ out_counts, double* __restrict__ pfirst, double* __restrict__ plast,
    const uint32_t* status) {
    if (*status != 0u) return;
    const int lane = lane_id();
    const int64_t chunk = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t i0 = chunk * kChunk;
    if (i0 >= n) return;
    const int cnt = (int)((n - i0) < kChunk ? (n - i0) : kChunk);
    const ChunkItem it = chunk_item(s, seg_id, seg_start, n, pos_bits, i0, cnt, lane);
    if (it.ends) out_counts[it.seg] = (int32_t)(i0 + lane + 1 - seg_start[it.seg]);

    const uintptr_t vmask = (uintptr_t)(V * sizeof(float)) - 1u;
    const bool vec = (V > 1) && (width % V == 0) &&
                     ((((uintptr_t)vals) | ((uintptr_t)out_vals)) & vmask) == 0;
    for (int64_t c0 = 0; c0 < width; c0 += (int64_t)kWave * V) {
        const int64_t col = c0 + (int64_t)lane * V;
        double acc[V];
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] = 0.0;
        for (int j0 = 0; j0 < cnt; j0 += 8) {
            float row[8][V];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + u;
                if (j < cnt) {
                    const uint32_t pos = read_lane(it.pos, j);
                    load_row<V>(row[u], vals + (int64_t)pos * width + col, col, width, vec);
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + u;
                if (j < cnt) {
#pragma unroll
                    for (int v = 0; v < V; ++v) acc[v] += (double)row[u][v];
                    const int kind = read_lane(it.kind, j);
                    if (kind != kFlushNone) {
                        if (kind == kFlushOut)
                            store_row<V>(out_vals + (int64_t)read_lane(it.seg, j) * width + col,
                                         acc, col, width, vec);
                        else if (kind == kFlushFirst)
                            store_part<V>(pfirst + chunk * width + col, acc, col, width);
                        else
                            store_part<V>(plast + chunk * width + col, acc, col, width);
#pragma unroll
                        for (int v = 0; v < V; ++v) acc[v] = 0.0;
                    }
                }
            }
        }
    }
}

// Width 1: one lookup per lane, segmented inclusive scan (double) across the wave.
__global__ __launch_bounds__(256) void k_dupsum_scalar(
    const uint64_t* __restrict__ s, const int32_t* __restrict__ seg_id,
    const int32_t* __restrict__ seg_start, int64_t n, int pos_bits,
    const float* __restrict__ vals, float* __restrict__ out_vals,
    int32_t* __restrict__ out_counts, double* __restrict__ pfirst, double* __restrict__ plast,
    const uint32_t* status) {
    if (*status != 0u) return;
    const int lane = lane_id();
    const int64_t chunk = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t i0 = chunk * kChunk;
    if (i0 >= n) return;
    const int cnt = (int)((n - i0) < kChunk ? (n - i0) : kChunk);
    const ChunkItem it = chunk_item(s, seg_id, seg_start, n, pos_bits, i0, cnt, lane);
    if (it.ends) out_counts[it.seg] = (int32_t)(i0 + lane + 1 - seg_start[it.seg]);
    double x = lane < cnt ? (double)vals[it.pos] : 0.0;
    const int prev_seg = __shfl_up(it.seg, 1, kWave);
    bool f = lane == 0 || prev_seg != it.seg;  // first lookup of its segment in this chunk
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const double y = __shfl_up(x, off, kWave);
        const bool g = __shfl_up((int)f, off, kWave) != 0;
        if (lane >= off && !f) {
            x = y + x;
            f = g;
        }
    }
    if (it.kind == kFlushOut)
        out_vals[it.seg] = (float)x;
    else if (it.kind == kFlushFirst)
        pfirst[chunk] = x;
    else if (it.kind == kFlushLast)
        plast[chunk] = x;
}

// Segments that cross chunk boundaries: the wave of the chunk where such a
// segment starts adds its partials in chunk order and rounds once.
template <int V>
__global__ __launch_bounds__(256) void k_dupsum_fixup(
    const int32_t* __restrict__ seg_id, const int32_t* __restrict__ seg_start, int64_t n,
    const double* __restrict__ pfirst, const double* __restrict__ plast, int64_t width,
    float* __restrict__ out_vals, const uint32_t* status) {
    if (*status != 0u) return;
    const int lane = lane_id();
    const int64_t chunk = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
    const int64_t i0 = chunk * kChunk;
    if (i0 >= n) return;
    const int64_t last = (i0 + kChunk < n ? i0 + kChunk : n) - 1;
    const int32_t seg = seg_id[last];
    const int64_t s0 = seg_start[seg], s1 = seg_start[seg + 1];
    if (!(s0 >= i0 && s1 > i0 + kChunk)) return;
    const int64_t ce = (s1 - 1) / kChunk;
    const uintptr_t vmask = (uintptr_t)(V * sizeof(float)) - 1u;
    const bool vec = (V > 1) && (width % V == 0) && (((uintptr_t)out_vals) & vmask) == 0;
    for (int64_t c0 = 0; c0 < width; c0 += (int64_t)kWave * V) {
        const int64_t col = c0 + (int64_t)lane * V;
        double acc[V], row[V];
        load_part<V>(acc, plast + chunk * width + col, col, width);
        for (int64_t c = chunk + 1; c <= ce; ++c) {
            load_part<V>(row, pfirst + c * width + col, col, width);
#pragma unroll
            for (int v = 0; v < V; ++v) acc[v] += row[v];
        }
        store_row<V>(out_vals + (int64_t)seg * width + col, acc, col, width, vec);
    }
}

// Finite check of the lookup values (SPOPT_VALIDATE).
__global__ void k_check_finite(const float* __restrict__ v, int64_t len, uint32_t* status) {
    bool bad = false;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < len;
         i += (int64_t)gridDim.x * blockDim.x)
        bad |= !finite_f(v[i]);
    if (ballot(bad) != 0ull && lane_id() == 0) atomicOr(status, kStatusNonFinite);
}

__global__ void k_write_i64(int64_t* p, int64_t v) { *p = v; }

int launch_status_clear(uint32_t* d_status, int nwords, hipStream_t s) {
    k_status_clear<<<1, 64, 0, s>>>(d_status, nwords);
    SPOPT_LAUNCHED();
    return SPOPT_OK;
}

}  // namespace spopt

using namespace spopt;

extern "C" int sparse_opt_workspace_size(int64_t n, int64_t width, int64_t key_space,
                                         size_t* bytes) {
    CanonLayout L;
    if (bytes == nullptr) return fail(SPOPT_EINVAL, "workspace_size: bytes is NULL");
    if (!canon_layout(n, width, key_space, &L))
        return fail(SPOPT_EINVAL, "workspace_size: bad n=%lld width=%lld key_space=%lld",
                    (long long)n, (long long)width, (long long)key_space);
    *bytes = L.total;
    return SPOPT_OK;
}

extern "C" int coo_from_lookups(const int64_t* ids, const float* vals, int64_t n, int64_t width,
                                int64_t key_space, int64_t* out_keys, float* out_vals,
                                int32_t* out_counts, int64_t* d_nunique, void* workspace,
                                size_t workspace_bytes, void* stream, uint32_t flags) {
    hipStream_t st = (hipStream_t)stream;
    CanonLayout L;
    if (n >= ((int64_t)1 << 31)) return fail(SPOPT_EOVERFLOW, "coo_from_lookups: n >= 2^31");
    if (!canon_layout(n, width, key_space, &L))
        return fail(SPOPT_EINVAL, "coo_from_lookups: bad n=%lld width=%lld key_space=%lld",
                    (long long)n, (long long)width, (long long)key_space);
    if (d_nunique == nullptr) return fail(SPOPT_EINVAL, "coo_from_lookups: d_nunique is NULL");
    if (n > 0 && (ids == nullptr || vals == nullptr || out_keys == nullptr ||
                  out_vals == nullptr || out_counts == nullptr))
        return fail(SPOPT_EINVAL, "coo_from_lookups: NULL array");
    if (workspace == nullptr || workspace_bytes < L.total)
        return fail(SPOPT_EWORKSPACE, "coo_from_lookups: workspace %zu bytes, need %zu",
                    workspace_bytes, L.total);
    char* ws = (char*)workspace;
    uint64_t* a = (uint64_t*)(ws + L.off_a);
    uint64_t* b = (uint64_t*)(ws + L.off_b);
    uint32_t* hist = (uint32_t*)(ws + L.off_hist);
    uint32_t* blk = (uint32_t*)(ws + L.off_blk);
    int32_t* seg_id = (int32_t*)(ws + L.off_segid);
    int32_t* seg_start = (int32_t*)(ws + L.off_segstart);
    double* pfirst = (double*)(ws + L.off_pfirst);
    double* plast = (double*)(ws + L.off_plast);
    uint32_t* status = (uint32_t*)(ws + L.off_status);

    if (n == 0) {
        k_write_i64<<<1, 1, 0, st>>>(d_nunique, 0);
        SPOPT_LAUNCHED();
        return SPOPT_OK;
    }
    int rc = launch_status_clear(status, 4, st);
    if (rc) return rc;
    const bool validate = (flags & SPOPT_VALIDATE) != 0;
    if (validate) {
        const int64_t len = n * width;
        const int grid = (int)(ceil_div(len, 256) < 4096 ? ceil_div(len, 256) : 4096);
        k_check_finite<<<grid, 256, 0, st>>>(vals, len, status);
        SPOPT_LAUNCHED();
    }

    // Radix sort on the id bits of the packed words.
    const uint32_t full_mask = kRadix - 1;
    auto pass_bits = [&](int p) {
        const int rem = L.key_bits - p * kRadixBits;
        return rem < kRadixBits ? rem : kRadixBits;
    };
    const int64_t nblk = L.nblk_sort;
    k_pack_hist<<<(unsigned)nblk, kSortThreads, 0, st>>>(
        ids, n, key_space, L.pos_bits, L.pos_bits, L.passes ? ((1u << pass_bits(0)) - 1u) : 0u,
        a, hist, nblk, L.passes > 0, status);
    SPOPT_LAUNCHED();
    if (validate) {
        uint32_t h_status = 0;
        SPOPT_HIP(hipMemcpyAsync(&h_status, status, sizeof(uint32_t), hipMemcpyDeviceToHost, st));
        SPOPT_HIP(hipStreamSynchronize(st));
        if (h_status != 0u) return status_to_code(h_status, "coo_from_lookups");
    }
    uint64_t* src = a;
    uint64_t* dst = b;
    for (int p = 0; p < L.passes; ++p) {
        const int shift = L.pos_bits + p * kRadixBits;
        const int nb = pass_bits(p);
        const uint32_t mask = (nb == kRadixBits) ? full_mask : ((1u << nb) - 1u);
        if (p > 0) {
            k_hist<<<(unsigned)nblk, kSortThreads, 0, st>>>(src, n, shift, mask, hist, nblk);
            SPOPT_LAUNCHED();
        }
        k_scan_u32<<<1, 1024, 0, st>>>(hist, (int64_t)kRadix * nblk);
        SPOPT_LAUNCHED();
        k_scatter<<<(unsigned)nblk, kSortThreads, 0, st>>>(src, dst, n, shift, mask, nb, hist,
                                                           nblk);
        SPOPT_LAUNCHED();
        uint64_t* t = src;
        src = dst;
        dst = t;
    }
    const uint64_t* sorted = src;

    // Segments.
    k_seg_count<<<(unsigned)L.nblk_seg, 256, 0, st>>>(sorted, n, L.pos_bits, blk);
    SPOPT_LAUNCHED();
    k_seg_scan<<<1, 1024, 0, st>>>(blk, L.nblk_seg, n, seg_start, d_nunique, status);
    SPOPT_LAUNCHED();
    k_seg_emit<<<(unsigned)L.nblk_seg, 256, 0, st>>>(sorted, n, L.pos_bits, blk, seg_id,
                                                     seg_start, out_keys, status);
    SPOPT_LAUNCHED();

    // Duplicate sums: 4 chunks (waves) per block.
    const unsigned grid = (unsigned)ceil_div(L.nchunks, 4);
    if (width == 1) {
        k_dupsum_scalar<<<grid, 256, 0, st>>>(sorted, seg_id, seg_start, n, L.pos_bits, vals,
                                              out_vals, out_counts, pfirst, plast, status);
        SPOPT_LAUNCHED();
        k_dupsum_fixup<1><<<grid, 256, 0, st>>>(seg_id, seg_start, n, pfirst, plast, 1, out_vals,
                                                status);
        SPOPT_LAUNCHED();
    } else if (width % 4 == 0 && width >= 256) {
        k_dupsum_rows<4><<<grid, 256, 0, st>>>(sorted, seg_id, seg_start, n, L.pos_bits, vals,
                                               width, out_vals, out_counts, pfirst, plast, status);
        SPOPT_LAUNCHED();
        k_dupsum_fixup<4><<<grid, 256, 0, st>>>(seg_id, seg_start, n, pfirst, plast, width,
                                                out_vals, status);
        SPOPT_LAUNCHED();
    } else if (width % 2 == 0 && width >= 128) {
        k_dupsum_rows<2><<<grid, 256, 0, st>>>(sorted, seg_id, seg_start, n, L.pos_bits, vals,
                                               width, out_vals, out_counts, pfirst, plast, status);
        SPOPT_LAUNCHED();
        k_dupsum_fixup<2><<<grid, 256, 0, st>>>(seg_id, seg_start, n, pfirst, plast, width,
                                                out_vals, status);
        SPOPT_LAUNCHED();
    } else {
        k_dupsum_rows<1><<<grid, 256, 0, st>>>(sorted, seg_id, seg_start, n, L.pos_bits, vals,
                                               width, out_vals, out_counts, pfirst, plast, status);
        SPOPT_LAUNCHED();
        k_dupsum_fixup<1><<<grid, 256, 0, st>>>(seg_id, seg_start, n, pfirst, plast, width,
                                                out_vals, status);
        SPOPT_LAUNCHED();
    }
    return SPOPT_OK;
}
