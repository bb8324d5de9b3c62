// csr_full.hpp - the blocks that build a full-row CSR's row_offsets and
// col_indices from ascending row ids.  Shared by csr_from_coo (its own launch)
// and by csr_from_lookups (the same blocks after the duplicate-sum combine, in
// one launch).  Included by one translation unit each; everything is static.
//
// Follows the optirs_gpu sparse_optimizer page, section "Sparse gradient
// representations": row_offsets[r] = cols * #{ids < r} for a CsrGradient whose
// touched rows are complete, col_indices 0..cols-1 for every touched row.
#pragma once
#include "common.hpp"

namespace spopt {

constexpr int kRoThreads = 256;

struct Bounds2 {
    int64_t b0, b1;
};

// Lower bounds of x0 and x1 in the ascending a[0, n), found by the whole block.
// Every block of the launch searches the same array, so the first round, whose
// probes are the same for all blocks and spaced too far apart to share cache
// lines, is kept to one wave's kWave probes, used for both targets.  Later
// rounds place kRoThreads * kLbPer probes in each target's interval, probe
// e * kRoThreads + tid on thread tid, so that one load instruction of a wave
// reads neighbouring entries: 65,536 entries take two dependent loads.  Probe positions stay below n_alloc
// (the array's length; n <= n_alloc is the count read from the device), so the
// first round's loads need not wait for n.  red: LDS, one row per wave.
constexpr int kLbPer = 4;

__device__ __forceinline__ Bounds2 block_lower_bounds2(const int64_t* __restrict__ a,
                                                       int64_t n_alloc, int64_t n, int64_t x0,
                                                       int64_t x1, uint32_t (*red)[4]) {
    if (n_alloc <= 0) return {0, 0};
    const int tid = (int)threadIdx.x, w = tid >> 6;
    const int64_t x[2] = {x0, x1};
    int64_t lo[2] = {0, 0}, hi[2] = {n_alloc, n_alloc};  // candidates [lo, min(hi, n))
    bool done[2] = {false, false};
    for (bool first = true;; first = false) {
        const int64_t probes = first ? kWave : (int64_t)kRoThreads * kLbPer;
        int64_t step[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t len = hi[j] - lo[j];
            step[j] = len <= probes ? 1 : (len + probes - 1) / probes;
        }
        uint32_t b[4] = {0u, 0u, 0u, 0u};  // this wave's counts: below x0, valid, below x1, valid
        if (first) {
            if (w == 0) {  // both intervals are [0, n_alloc): one set of probes
                const int64_t q = (int64_t)(tid + 1) * step[0] - 1;
                const bool in = q < hi[0];
                const int64_t v = a[in ? q : 0];
                const bool valid = in && q < n;
                b[0] = (uint32_t)popc64(ballot(valid && v < x[0]));
                b[1] = (uint32_t)popc64(ballot(valid));
                b[2] = (uint32_t)popc64(ballot(valid && v < x[1]));
                b[3] = b[1];
            }
        } else {
            int64_t q[2][kLbPer], v[2][kLbPer];
            bool in[2][kLbPer];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < kLbPer; ++e) {
                    q[j][e] = lo[j] + (int64_t)(e * kRoThreads + tid + 1) * step[j] - 1;
                    in[j][e] = !done[j] && q[j][e] < hi[j];
                    v[j][e] = a[in[j][e] ? q[j][e] : 0];
                }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int e = 0; e < kLbPer; ++e) {
                    const bool valid = in[j][e] && q[j][e] < n;
                    b[2 * j] += (uint32_t)popc64(ballot(valid && v[j][e] < x[j]));
                    b[2 * j + 1] += (uint32_t)popc64(ballot(valid));
                }
        }
        if (lane_id() == 0) {
#pragma unroll
            for (int k = 0; k < 4; ++k) red[w][k] = b[k];
        }
        __syncthreads();
        int64_t c[2] = {0, 0}, nv[2] = {0, 0};
#pragma unroll
        for (int k = 0; k < kRoThreads / kWave; ++k) {
            c[0] += red[k][0]; nv[0] += red[k][1];
            c[1] += red[k][2]; nv[1] += red[k][3];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (!done[j] && step[j] == 1) {
                lo[j] += c[j];
                done[j] = true;
            } else if (!done[j]) {
                // Probes before c are below x: the bound is at least lo + c*step.
                // Probe c (if valid) is not: the bound is at most its position.
                const int64_t nlo = lo[j] + c[j] * step[j];
                hi[j] = c[j] < nv[j] ? lo[j] + (c[j] + 1) * step[j] - 1 : (hi[j] < n ? hi[j] : n);
                lo[j] = nlo;
                done[j] = hi[j] <= lo[j];
            }
        }
        if (done[0] && done[1]) return {lo[0], lo[1]};
    }
}

// Full-row COO (keys are row ids, each row complete): row_offsets[r] =
// cols * #{keys < r}.  A row block owns kRoBits consecutive entries: it finds
// the keys in its rows with one block-wide search for both bounds (or reads
// them from a table of per-block counts), flags them
// in LDS, packs the flags into a bitmap and turns it into prefix counts with
// popcounts; each thread then writes four consecutive offsets per 16-byte
// store (VEC, chosen on the host when row_offsets is 16-byte aligned).  The
// first nblk_ci blocks write col_indices (0..cols-1 per touched row,
// cols % 4 == 0).  Both are streamed out with nontemporal stores: tens of MB
// that the update does not read back (it reads two offsets per touched row and
// no column index of a full row) would otherwise displace cached lines.
constexpr int kRoBits = 8192;
constexpr int kRoDense = kRoBits / kRoThreads;  // key loads in flight per thread, dense blocks
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));


// Column block cb of ncb: col_indices of nnz full rows (cols % 4 == 0, the
// array 16-byte aligned).  nnz * cols < 2^31 (checked on the host), so 32-bit
// column arithmetic.
__device__ __forceinline__ void csr_col_block(int64_t cb, int64_t ncb, int64_t nnz, int64_t cols,
                                              int32_t* __restrict__ col_indices) {
    const uint32_t total4 = (uint32_t)(nnz * cols / 4);
    const uint32_t ucols = (uint32_t)cols;
    const uint32_t stride = (uint32_t)ncb * kRoThreads;
    for (uint32_t q = (uint32_t)cb * kRoThreads + threadIdx.x; q < total4; q += stride) {
        const int32_t c = (int32_t)((q * 4u) % ucols);
        const i32x4 cv = {c, c + 1, c + 2, c + 3};
        __builtin_nontemporal_store(cv, reinterpret_cast<i32x4*>(col_indices) + q);
    }
}

// Row block rb: row_offsets[rb * kRoBits, min(rb * kRoBits + kRoBits, rows + 1)).
// keys: nnz ascending row ids (nnz_host the array's length).  bnd: NULL to
// search the keys, else bnd[b] = #{keys < b * kRoBits} for every block b.
template <bool VEC>
__device__ __forceinline__ void csr_row_block(int64_t rb, const int64_t* __restrict__ keys,
                                              int64_t nnz_host, int64_t nnz, int64_t rows,
                                              int64_t cols, int32_t* __restrict__ row_offsets,
                                              const int32_t* bnd) {
    constexpr int kWordsPer = kRoBits / (32 * kRoThreads);  // bitmap words per thread
    static_assert(kWordsPer >= 1 && kRoBits == 32 * kRoThreads * kWordsPer, "whole words");
    __shared__ uint4 flags[kRoBits / 16];  // one byte per row of the block
    __shared__ uint32_t bits[kRoBits / 32];
    __shared__ uint32_t wpre[kRoBits / 32];
    __shared__ uint32_t red[kRoThreads / kWave][4];
    __shared__ uint32_t wt[kRoThreads / kWave];
    const int tid = (int)threadIdx.x;
    const int64_t r0 = rb * kRoBits;
    const int64_t r1 = (r0 + kRoBits < rows + 1) ? r0 + kRoBits : rows + 1;
#pragma unroll
    for (int j = 0; j < 2 * kWordsPer; ++j) flags[j * kRoThreads + tid] = make_uint4(0u, 0u, 0u, 0u);
    // Every flag is zeroed before any thread sets one (a thread's zeroing of
    // its slice must not land after another thread's flag in it).
    __syncthreads();
    int64_t ka, kb;
    if (bnd != nullptr) {
        // #keys below the block's first row and below the next block's, as
        // recorded while the keys were numbered; clamped to nnz, so a table
        // left unwritten (a call that failed, U = 0) gives empty rows.
        const int64_t nblk = rows / kRoBits + 1;
        const int64_t a = bnd[rb], b = rb + 1 < nblk ? bnd[rb + 1] : nnz;
        ka = a < 0 ? 0 : (a < nnz ? a : nnz);
        kb = b < ka ? ka : (b < nnz ? b : nnz);
    } else {
        const Bounds2 bd = block_lower_bounds2(keys, nnz_host, nnz, r0, r1, red);
        ka = bd.b0;
        kb = bd.b1;
    }
    // Keys in [ka, kb) lie in [r0, r0 + kRoBits) for canonical input, so the
    // low 32 bits of key - r0 are its offset; the bound test keeps malformed
    // trusted input inside the block's rows.  Each key sets its row's byte
    // flag with a plain store: neighbouring keys of the block of the most
    // popular rows would collide lane against lane in atomics on a bitmap.
    // That block holds thousands of keys, loaded kRoDense per thread (wave
    // instructions over consecutive keys) before any is used.
    const uint32_t* lowk = reinterpret_cast<const uint32_t*>(keys);  // little endian
    const uint32_t ur0 = (uint32_t)r0;
    uint8_t* fbyte = reinterpret_cast<uint8_t*>(flags);
    if (kb - ka <= kRoThreads) {
        const int64_t k = ka + tid;
        if (k < kb) {
            const uint32_t o = lowk[2 * k] - ur0;
            if (o < (uint32_t)kRoBits) fbyte[o] = 1u;
        }
    } else {
        for (int64_t k0 = ka + tid; k0 < kb; k0 += (int64_t)kRoDense * kRoThreads) {
            uint32_t x[kRoDense];
#pragma unroll
            for (int j = 0; j < kRoDense; ++j) {
                const int64_t k = k0 + (int64_t)j * kRoThreads;
                x[j] = lowk[2 * (k < kb ? k : k0)];
            }
#pragma unroll
            for (int j = 0; j < kRoDense; ++j) {
                const uint32_t o = x[j] - ur0;
                if (k0 + (int64_t)j * kRoThreads < kb && o < (uint32_t)kRoBits) fbyte[o] = 1u;
            }
        }
    }
    __syncthreads();
    // Thread t packs the flags of rows 32w .. 32w+31 into bitmap word w for its
    // kWordsPer consecutive words (byte i of a little-endian word is bits
    // 8i .. 8i+7), then the words are scanned.
    auto nib = [](uint32_t d) -> uint32_t {
        return (d & 1u) | ((d >> 7) & 2u) | ((d >> 14) & 4u) | ((d >> 21) & 8u);
    };
    uint32_t cnt[kWordsPer], sum = 0;
#pragma unroll
    for (int j = 0; j < kWordsPer; ++j) {
        const int wi = tid * kWordsPer + j;
        const uint4 fa = flags[2 * wi], fb = flags[2 * wi + 1];
        const uint32_t word = nib(fa.x) | nib(fa.y) << 4 | nib(fa.z) << 8 | nib(fa.w) << 12 |
                              nib(fb.x) << 16 | nib(fb.y) << 20 | nib(fb.z) << 24 | nib(fb.w) << 28;
        bits[wi] = word;
        cnt[j] = (uint32_t)__popc(word);
        sum += cnt[j];
    }
    uint32_t total;
    uint32_t run = block_excl_scan(sum, wt, &total);
#pragma unroll
    for (int j = 0; j < kWordsPer; ++j) {
        wpre[tid * kWordsPer + j] = run;
        run += cnt[j];
    }
    __syncthreads();
    const int len = (int)(r1 - r0);
    if (VEC) {
        // Quads of rows: all four rows of a quad share one bitmap word.
        for (int o = 4 * (int)threadIdx.x; o < len; o += 4 * kRoThreads) {
            const uint32_t word = bits[o >> 5], pre = wpre[o >> 5];
            const int sh = o & 31;
            int32_t out[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[e] = (int32_t)((ka + (int64_t)(pre + (uint32_t)__popc(word & ((1u << (sh + e)) - 1u)))) * cols);
            if (o + 4 <= len) {
                const i32x4 q = {out[0], out[1], out[2], out[3]};
                __builtin_nontemporal_store(q, reinterpret_cast<i32x4*>(row_offsets + r0 + o));
            } else {
                for (int e = 0; e < len - o; ++e) row_offsets[r0 + o + e] = out[e];
            }
        }
    } else {
        for (int o = (int)threadIdx.x; o < len; o += kRoThreads) {
            const uint32_t below = wpre[o >> 5] + (uint32_t)__popc(bits[o >> 5] & ((1u << (o & 31)) - 1u));
            row_offsets[r0 + o] = (int32_t)((ka + (int64_t)below) * cols);
        }
    }
}

}  // namespace spopt
