// canon.hip - raw lookups -> canonical COO on the GPU (coo_from_lookups), and
// on to the full-row CSR in the same call (csr_from_lookups).
//
// Computes what the DiskSparseAdam README calls "Safe Duplicate Aggregation &
// Sorted I/O" (duplicates summed, indices sorted) and what the optirs_gpu
// sparse_optimizer page requires of a CooGradient (strictly ascending
// indices):
//   1. pack each lookup as (id << pos_bits) | position and radix-sort the
//      packed words on the id bits only (LSD, stable, so equal ids keep
//      lookup order, digits of at most 9 bits): one kernel counts the digits
//      of every pass, then each pass is one kernel whose tiles find their
//      offsets by decoupled look-back;
//   2. one kernel per tile of 256 sorted lookups: segment heads (id differs
//      from its predecessor) numbered by decoupled look-back, distinct ids and
//      counts emitted, and each segment's value rows summed in double in
//      sorted (= lookup) order and rounded once; segments that cross waves are
//      combined inside the tile in wave order;
//   3. segments that cross tiles leave double partial sums, which a second
//      kernel adds in tile order.  No atomics in any sum, so the result is the
//      same run to run.
// csr_from_lookups runs 1 and 2 (the segment kernel also recording how many
// ids lie below each 8192-row block), then one launch that does 3 and builds
// the CSR's row_offsets and col_indices (csr_full.hpp) from those counts.
// sparse_step_from_lookups runs 1 and 2 the same way and leaves 3 and the CSR
// blocks to the launch that updates the table (update.hip).
#include <stdarg.h>
#include <stdio.h>


#include "common.hpp"
#include "csr_full.hpp"
#include "seg_combine.hpp"

namespace spopt {

constexpr int kThreads = 256;
constexpr int kIpt = 2;                         // items per thread (radix passes)
constexpr int kSortThreads = 1024;              // threads of a radix-pass block
constexpr int kSortWaves = kSortThreads / kWave;
constexpr int kTile = kSortThreads * kIpt;      // lookups per radix-pass tile
constexpr int kRadixBits = 9;                   // at most 512 buckets per radix pass
constexpr int kRadix = 1 << kRadixBits;
constexpr int kMaxPasses = 8;
constexpr int kFixWaves2 = 16;                  // waves of the combining block
// Per-block key counts for csr_from_lookups are kept for tables of fewer rows.
constexpr int64_t kBndMaxRows = ((int64_t)1 << 31) - 1;

// Decoupled look-back.  A tile publishes one 32-bit word per count:
// bits 31..30 its state (aggregate of this tile / inclusive prefix through
// this tile), bits 29..0 the count, so n stays below 2^30.  Each word carries
// its own state and is written and read with device-coherent atomics, so no
// fence is needed.
constexpr uint32_t kLbAgg = 1u << 30;
constexpr uint32_t kLbInc = 2u << 30;
constexpr uint32_t kLbState = 3u << 30;
constexpr uint32_t kLbCount = (1u << 30) - 1u;
// Tiles are numbered by an atomic ticket, in the order blocks start, so a
// tile waits only for tiles that are already running and publish their own
// counts before they wait on anybody; the bound only turns a bug into a
// reported error instead of a hang.  Each round of a wait is a device-scope
// load (about a microsecond) and a short sleep, so 2^20 rounds outlast any
// plausible descheduling of the awaited block (about a second).
constexpr uint32_t kSpinLimit = 1u << 20;
// The pack kernel: at most this many blocks, each counting the digits of its
// share of the lookups into its own histograms (plain stores, nothing to zero
// beforehand); every radix pass sums them.  kPackIpt lookups per thread are
// loaded before any is used.
constexpr int kPackBlocks = 32;
constexpr int kPackIpt = 8;
// Up to this many radix tiles, the first pass reads the per-tile digit counts
// the pack kernel wrote instead of looking back; kCountBatch counts are loaded
// per round trip.  (Later passes would need their tiles' counts from the pass
// before: added up with a global atomic per key they took 24 µs a pass;
// counted in LDS per source tile and stored as prefixes, they cost the pass
// that writes them about as much as they save the pass that reads them.)
constexpr int kMaxCountTiles = 64;
constexpr int kCountBatch = 32;

struct CanonLayout {
    int key_bits, pos_bits, passes, digit_bits;
    int radix;  // row width of the digit counts: 2^digit_bits, at least one wave
    int64_t ntiles, nsum;
    int64_t npack;  // blocks of the pack kernel
    size_t off_a, off_b, off_part, off_pflag, off_thist0, off_clear, clear_bytes, off_status,
        off_tickets,
        off_sumwords, off_words, off_segstart, off_tcross, off_tfirst, off_tlast, off_bnd,
        bnd_entries, total;
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
    // As few passes as digits of at most 9 bits allow, digits as even as
    // possible (24-bit keys: three passes of 8; 26-bit keys: three of 9, not
    // four of 7).  The 512 buckets of a 9-bit digit are owned by half of a
    // pass block's 1024 threads.  (Wider digits would need fewer passes still,
    // but then every thread owns several digits, and the look-back words are
    // device-coherent atomics, which do not coalesce: 1024 or 4096 buckets
    // per tile cost more per pass than the passes they save.)
    L->passes = (L->key_bits + kRadixBits - 1) / kRadixBits;
    L->digit_bits = L->passes ? (L->key_bits + L->passes - 1) / L->passes : 0;
    // A pass's digits are owned by whole waves, so a row of counts or
    // look-back words is at least 64 wide (digits past 2^digit_bits count 0).
    L->radix = (1 << L->digit_bits) > kWave ? (1 << L->digit_bits) : kWave;
    L->ntiles = ceil_div(n, kTile);
    L->nsum = ceil_div(n, kSumTile);
    L->npack = ceil_div(n, (int64_t)kPackIpt * kThreads);
    if (L->npack > kPackBlocks) L->npack = kPackBlocks;
    if (L->npack < 1) L->npack = 1;
    const size_t P = (size_t)(L->passes ? L->passes : 1);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes, 256);
        return at;
    };
    L->off_a = take(sizeof(uint64_t) * (size_t)n);
    L->off_b = take(sizeof(uint64_t) * (size_t)n);
    // Digit histograms and range flag of each pack block.
    L->off_part = take(sizeof(uint32_t) * (size_t)kPackBlocks * (size_t)L->radix * P);
    L->off_pflag = take(sizeof(uint32_t) * (size_t)kPackBlocks);
    // Digit counts of each radix tile for the first pass (written whole by the
    // pack kernel when the tiles are few).
    L->off_thist0 = take(sizeof(uint32_t) * (size_t)L->radix * (size_t)L->ntiles);
    // Everything the kernels after the pack kernel must find zeroed sits in
    // one contiguous region, which the pack kernel zeroes.
    L->off_clear = o;
    L->off_status = take(sizeof(uint32_t) * 4);
    // tickets: one per radix pass and the segment-and-sum kernel's.
    L->off_tickets = take(sizeof(uint32_t) * (kMaxPasses + 1));
    L->off_words = take(sizeof(uint32_t) * (size_t)L->radix * (size_t)L->ntiles * P);
    L->off_sumwords = take(sizeof(uint32_t) * (size_t)L->nsum);
    L->clear_bytes = o - L->off_clear;
    L->off_segstart = take(sizeof(int32_t) * ((size_t)n + 1));
    L->off_tcross = take(sizeof(int32_t) * (size_t)L->nsum);
    L->off_tfirst = take(sizeof(double) * (size_t)L->nsum * (size_t)width);
    L->off_tlast = take(sizeof(double) * (size_t)L->nsum * (size_t)width);
    // #ids below each kRoBits-row block of a key_space-row table (csr_from_lookups).
    L->bnd_entries = key_space <= kBndMaxRows ? (size_t)(key_space / kRoBits + 1) : 0;
    L->off_bnd = take(sizeof(int32_t) * L->bnd_entries);
    L->total = o;
    return true;
}

__device__ __forceinline__ uint32_t ld_dev(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits for a look-back word to leave state 0.  Returns false on timeout.
__device__ __forceinline__ bool lb_wait(const uint32_t* p, uint32_t* out) {
    for (uint32_t spins = 0; spins < kSpinLimit; ++spins) {
        const uint32_t v = ld_dev(p);
        if (v & kLbState) {
            *out = v;
            return true;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

// Sum of the counts published by tiles tile-1, tile-2, ... (words at
// lb[j * stride]) back to the nearest inclusive prefix.  Reads kLookDepth
// words at a time so that one memory round trip covers that many
// predecessors: every tile starts at once, so inclusive prefixes are still
// scarce when most tiles look back.
constexpr int kLookDepth = 4;
__device__ __forceinline__ bool look_back(const uint32_t* lb, int64_t tile, int64_t stride,
                                          uint32_t* excl_out) {
    uint32_t excl = 0;
    int64_t j = tile - 1;
    while (j >= 0) {
        uint32_t v[kLookDepth];
#pragma unroll
        for (int u = 0; u < kLookDepth; ++u)
            v[u] = (j - u >= 0) ? ld_dev(lb + (j - u) * stride) : kLbInc;
#pragma unroll
        for (int u = 0; u < kLookDepth; ++u) {
            if (j - u < 0) {
                *excl_out = excl;
                return true;
            }
            uint32_t x = v[u];
            if (!(x & kLbState) && !lb_wait(lb + (j - u) * stride, &x)) return false;
            excl += x & kLbCount;
            if ((x & kLbState) == kLbInc) {
                *excl_out = excl;
                return true;
            }
        }
        j -= kLookDepth;
    }
    *excl_out = excl;
    return true;
}

__global__ void k_status_clear(uint32_t* st, int nwords) {
    if ((int)threadIdx.x < nwords) st[threadIdx.x] = 0u;
}

// ------------------------------------------------------------------ sort ---

// Range-check ids, pack (id << pos_bits | position), and count the digits of
// every radix pass, in LDS first.  The grid (at most kPackBlocks blocks)
// strides over the lookups; block g writes its histograms to part[g] and its
// range flag to pflag[g] with plain stores.  The blocks also zero the region
// the later kernels of the call need zeroed (status, tickets, look-back
// words): those kernels start after this one has ended.
__global__ __launch_bounds__(kThreads) void k_pack(const int64_t* __restrict__ ids, int64_t n,
                                                   int64_t key_space, int pos_bits, int passes,
                                                   int digit_bits, int radix,
                                                   uint64_t* __restrict__ out,
                                                   uint32_t* __restrict__ part,
                                                   uint32_t* __restrict__ pflag,
                                                   uint4* __restrict__ zero, int64_t nzero16,
                                                   uint32_t* __restrict__ thist0) {
    static_assert((int64_t)kPackIpt * kThreads == kTile, "a pack chunk is a radix tile");
    static_assert(kRadix % kThreads == 0, "threads own whole digits of a chunk's counts");
    __shared__ uint32_t h[kMaxPasses * kRadix];
    __shared__ uint32_t h0[kRadix];
    const int tid = threadIdx.x;
    const int words = passes * radix;  // radix: row width of the counts, <= kRadix
    for (int i = tid; i < words; i += kThreads) h[i] = 0;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + tid; i < nzero16;
         i += (int64_t)gridDim.x * kThreads)
        zero[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    const uint32_t dmask = (1u << digit_bits) - 1u;
    bool bad = false;
    constexpr int64_t kChunk = (int64_t)kPackIpt * kThreads;
    const int64_t stride = (int64_t)gridDim.x * kChunk;
    for (int64_t base = (int64_t)blockIdx.x * kChunk; base < n; base += stride) {
        int64_t id[kPackIpt];
#pragma unroll
        for (int j = 0; j < kPackIpt; ++j) {
            const int64_t i = base + (int64_t)j * kThreads + tid;
            id[j] = ids[i < n ? i : n - 1];
        }
        if (thist0 != nullptr) {  // this chunk's first-digit counts (thread t: digits t + k*256)
            for (int d = tid; d < radix; d += kThreads) h0[d] = 0u;
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < kPackIpt; ++j) {
            const int64_t i = base + (int64_t)j * kThreads + tid;
            if (i < n) {
                int64_t x = id[j];
                if (x < 0 || x >= key_space) {
                    bad = true;
                    x = 0;  // keep sorting a safe key; the result is discarded
                }
                const uint64_t packed = ((uint64_t)x << pos_bits) | (uint64_t)i;
                out[i] = packed;
                for (int p = 0; p < passes; ++p)
                    atomicAdd(&h[p * radix +
                                 ((uint32_t)(packed >> (pos_bits + p * digit_bits)) & dmask)],
                              1u);
                if (thist0 != nullptr && passes > 0)
                    atomicAdd(&h0[(uint32_t)(packed >> pos_bits) & dmask], 1u);
            }
        }
        if (thist0 != nullptr) {
            __syncthreads();
            for (int d = tid; d < radix; d += kThreads)  // read and later zeroed by tid
                thist0[(base / kChunk) * radix + d] = h0[d];
        }
    }
    const bool any_bad = __syncthreads_or(bad);
    uint32_t* mine = part + (int64_t)blockIdx.x * words;
    for (int i = tid; i < words; i += kThreads) mine[i] = h[i];
    if (tid == 0) pflag[blockIdx.x] = any_bad ? kStatusRange : 0u;
}

// One stable radix pass (digits of nbits <= 9 bits) in a single kernel.  A
// block takes the next tile ticket, ranks its kTile items (wave w owns items
// [w*128, (w+1)*128) in two rounds of 64: lanes holding the same digit are
// matched with one ballot per digit bit, a lane's rank is the number of lower
// lanes with its digit plus the wave's running count of that digit), and
// thread d < 2^nbits publishes the tile's count of digit d and sums the counts
// of the tiles before it by decoupled look-back.  Its items then go to
// digit base (scan of the pass histogram) + prefix of the tiles before +
// prefix of the waves before + rank.
__global__ __launch_bounds__(kSortThreads) void k_onesweep(
    const uint64_t* __restrict__ in, uint64_t* __restrict__ out, int64_t n, int shift, int nbits,
    int radix, const uint32_t* __restrict__ part, int npack, int part_stride, const uint32_t* pflag,
    uint32_t* lb, uint32_t* ticket, uint32_t* status, const uint32_t* __restrict__ thist) {
    static_assert(kSortThreads >= kRadix && kRadix % kWave == 0,
                  "threads 0..kRadix-1 own the digits (whole waves)");
    __shared__ uint32_t cnt[kSortWaves][kRadix];
    __shared__ uint32_t base[kRadix];
    __shared__ uint32_t wt[kSortWaves];
    __shared__ uint32_t s_tile, s_bad;
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = lane_id();
    // thist (first pass, few tiles): the digit counts of every tile, so tile =
    // block and no look-back; else tiles by ticket and decoupled look-back.
    if (tid == 0) {
        if (thist == nullptr) s_tile = atomicAdd(ticket, 1u);
        s_bad = 0u;
    }
    for (int i = tid; i < kSortWaves * kRadix; i += kSortThreads) (&cnt[0][0])[i] = 0;
    __syncthreads();
    const int64_t tile = thist != nullptr ? (int64_t)blockIdx.x : (int64_t)s_tile;
    // Threads below the pass's digit count own the digits (at least a whole
    // wave, so ownership is wave-uniform; digits past 2^nbits count nothing).
    const bool owner = tid < ((1 << nbits) > kWave ? (1 << nbits) : kWave);

    const int64_t first = tile * kTile + (int64_t)w * (kIpt * kWave);
    const uint64_t lt = lanemask_lt();
    uint64_t key[kIpt];
    uint32_t dig[kIpt], rank[kIpt];
    bool valid[kIpt];
#pragma unroll
    for (int r = 0; r < kIpt; ++r) {
        const int64_t i = first + (int64_t)r * kWave + lane;
        valid[r] = i < n;
        key[r] = valid[r] ? in[i] : 0ull;
        dig[r] = (uint32_t)(key[r] >> shift) & ((1u << nbits) - 1u);
    }
    // This pass's count of digit tid: the sum of the pack blocks' counts,
    // loaded after the keys (loads complete in order, so the ranking below
    // waits for the keys only) and needed only after the look-back.
    uint32_t hpart[kPackBlocks];
    if (owner) {
#pragma unroll
        for (int g = 0; g < kPackBlocks; ++g)
            hpart[g] = part[(int64_t)(g < npack ? g : 0) * part_stride + tid];
    }
    // Counts of digit tid in the first kCountBatch tiles before this one.
    uint32_t tpre[kCountBatch];
    if (owner && thist != nullptr) {
#pragma unroll
        for (int g = 0; g < kCountBatch; ++g)
            tpre[g] = thist[(int64_t)(g < tile ? g : 0) * radix + tid];
    }
#pragma unroll
    for (int r = 0; r < kIpt; ++r) {
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

    // Thread d owns digit d: prefix over the waves, then over earlier tiles.
    const int d = tid;
    uint32_t excl = 0, hd = 0;
    if (owner) {
        uint32_t run = 0;
        for (int ww = 0; ww < kSortWaves; ++ww) {
            const uint32_t c = cnt[ww][d];
            cnt[ww][d] = run;
            run += c;
        }
        bool ok = true;
        if (thist != nullptr) {
#pragma unroll
            for (int g = 0; g < kCountBatch; ++g) excl += g < tile ? tpre[g] : 0u;
            for (int64_t g0 = kCountBatch; g0 < tile; g0 += kCountBatch) {
                uint32_t more[kCountBatch];
#pragma unroll
                for (int g = 0; g < kCountBatch; ++g)
                    more[g] = thist[(g0 + g < tile ? g0 + g : 0) * radix + d];
#pragma unroll
                for (int g = 0; g < kCountBatch; ++g) excl += g0 + g < tile ? more[g] : 0u;
            }
        } else {
            uint32_t* mine = lb + tile * radix + d;
            if (tile == 0) {
                st_dev(mine, kLbInc | run);
            } else {
                st_dev(mine, kLbAgg | run);
                ok = look_back(lb + d, tile, radix, &excl);
                if (ok) st_dev(mine, kLbInc | (excl + run));
            }
        }
        if (!ok) atomicOr(&s_bad, 1u);
#pragma unroll
        for (int g = 0; g < kPackBlocks; ++g) hd += g < npack ? hpart[g] : 0u;
    }
    uint32_t total;
    const uint32_t gbase = block_excl_scan(hd, wt, &total);  // all threads; zeros past the owners
    if (owner) base[d] = gbase + excl;
    __syncthreads();
    if (s_bad) {
        if (tid == 0) atomicOr(status, kStatusTimeout);
        return;
    }
#pragma unroll
    for (int r = 0; r < kIpt; ++r) {
        if (!valid[r]) continue;
        const uint64_t dst = (uint64_t)base[dig[r]] + cnt[w][dig[r]] + rank[r];
        if (dst < (uint64_t)n) out[dst] = key[r];
    }
    // First pass: the pack blocks' range flags go to the status word, by the
    // last tile (no tile waits on it), for the kernels after this one.
    if (pflag != nullptr && tile == (int64_t)gridDim.x - 1 && tid < npack && pflag[tid] != 0u)
        atomicOr(status, kStatusRange);
}

// ------------------------------------------------------------- segments ---

// Run by one whole wave of tile `tile`: publishes `count` for the tile and
// returns in *excl the sum of the counts of all earlier tiles.  Each round
// trip reads the words of the 512 tiles below lo (lane l, load k: tile
// lo-1-l-64k) and sums them back to the nearest inclusive prefix or the
// nearest tile that has not published yet, then waits for that one.  Deep
// rounds matter because every tile starts at once: inclusive prefixes spread
// back-to-front only as fast as tiles finish their own look-back.  False on
// timeout.
__device__ __forceinline__ bool tile_exclusive_prefix(uint32_t* words, int64_t tile,
                                                      uint32_t count, uint32_t* excl_out) {
    constexpr int kDeep = 8;
    const int lane = lane_id();
    uint32_t excl = 0;
    bool ok = true;
    if (tile == 0) {
        if (lane == 0) st_dev(words, kLbInc | count);
    } else {
        if (lane == 0) st_dev(words + tile, kLbAgg | count);
        int64_t lo = tile;  // tiles [lo, tile) summed
        uint32_t spins = 0;
        while (lo > 0) {
            uint32_t v[kDeep];
#pragma unroll
            for (int k = 0; k < kDeep; ++k) {
                const int64_t tj = lo - 1 - lane - (int64_t)k * kWave;
                v[k] = tj >= 0 ? ld_dev(words + tj) : kLbInc;  // below tile 0: a zero prefix
            }
            bool done = false;
            int64_t advanced = 0;
#pragma unroll
            for (int k = 0; k < kDeep; ++k) {
                if (!done) {
                    const int64_t base = lo - 1 - (int64_t)k * kWave;  // tile read by lane 0
                    const bool valid = base - lane >= 0;
                    const uint32_t x = valid ? v[k] : kLbInc;
                    const uint64_t not_ready = ballot(valid && (x & kLbState) == 0u);
                    const uint64_t inclusive = ballot(!valid || (x & kLbState) == kLbInc);
                    const int first_nr = not_ready ? __builtin_ctzll(not_ready) : kWave;
                    const int first_inc = inclusive ? __builtin_ctzll(inclusive) : kWave;
                    const int take = first_inc < first_nr ? first_inc + 1 : first_nr;
                    uint32_t part = (lane < take && valid) ? (x & kLbCount) : 0u;
#pragma unroll
                    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, kWave);
                    excl += part;
                    advanced += take;
                    if (first_inc < first_nr) {
                        lo = 0;  // reached an inclusive prefix (or tile 0's base)
                        done = true;
                    } else if (take < kWave) {
                        done = true;  // stopped at a tile that has not published
                    }
                }
            }
            if (lo == 0) break;
            lo -= advanced;
            if (advanced == 0) {
                if (++spins > kSpinLimit) {
                    ok = false;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        if (lane == 0 && ok) st_dev(words + tile, kLbInc | (excl + count));
    }
    *excl_out = excl;
    return ok;
}

// ----------------------------------------------------------- dup sums ---

// V-wide access to a row of floats.  V > 1 is chosen on the host only when the
// width is a multiple of V and the arrays are V*4-byte aligned, so a lane
// whose first column is inside the row owns all V of its columns.
// Straight-line: a lane past the end of the row loads the row's first V
// columns instead and zeroes them, so loads are never behind a branch.  The
// 16-byte form is a nontemporal load: each lookup's row is read once a step,
// and the hint keeps those rows from displacing lines that are read again.
template <int V>
__device__ __forceinline__ void load_row(float (&r)[V], const float* row, int64_t col,
                                         int64_t width) {
    const bool in = col < width;
    const float* src = row + (in ? col : 0);
    if constexpr (V == 4) {
        typedef float g4 __attribute__((ext_vector_type(4)));
        const g4 x = __builtin_nontemporal_load(reinterpret_cast<const g4*>(src));
        r[0] = in ? x.x : 0.f; r[1] = in ? x.y : 0.f; r[2] = in ? x.z : 0.f; r[3] = in ? x.w : 0.f;
    } else if constexpr (V == 2) {
        const float2 x = *reinterpret_cast<const float2*>(src);
        r[0] = in ? x.x : 0.f; r[1] = in ? x.y : 0.f;
    } else {
        const float x = src[0];
        r[0] = in ? x : 0.f;
    }
}

template <int V>
__device__ __forceinline__ void store_row_f(float* dst, const float (&r)[V], int64_t col,
                                            int64_t width) {
    if (col < width) {
        if constexpr (V == 4) {
            *reinterpret_cast<float4*>(dst) = make_float4(r[0], r[1], r[2], r[3]);
        } else if constexpr (V == 2) {
            *reinterpret_cast<float2*>(dst) = make_float2(r[0], r[1]);
        } else {
            dst[0] = r[0];
        }
    }
}

template <int V>
__device__ __forceinline__ void store_part(double* dst, const double (&r)[V], int64_t col,
                                           int64_t width) {
#pragma unroll
    for (int v = 0; v < V; ++v)
        if (col + v < width) dst[v] = r[v];
}

// Destination of the running sum when lookup j of a chunk closes it.
enum : int { kFlushNone = 0, kFlushOut = 1, kFlushFirst = 2, kFlushLast = 3 };

// Head count of every segment tile of kSumTile sorted lookups: the lookups
// whose id differs from their predecessor's, stored with a plain store.  When
// the tiles are few, k_seg_sum sums the counts of the tiles before its own in
// place of a look-back.
__global__ __launch_bounds__(kSumTile) void k_head_count(const uint64_t* __restrict__ s, int64_t n,
                                                        int pos_bits,
                                                        uint32_t* __restrict__ counts) {
    __shared__ uint32_t wc[kSumTile / kWave];
    const int64_t i = (int64_t)blockIdx.x * kSumTile + threadIdx.x;
    const int64_t ic = i < n ? i : n - 1;
    const uint64_t key = s[ic], prev = s[ic > 0 ? ic - 1 : 0];
    const bool head = i < n && (ic == 0 || (prev >> pos_bits) != (key >> pos_bits));
    const uint32_t c = (uint32_t)popc64(ballot(head));
    if (lane_id() == 0) wc[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
#pragma unroll
        for (int w = 0; w < kSumTile / kWave; ++w) t += wc[w];
        counts[blockIdx.x] = t;
    }
}

// Segments and their sums in one pass over the sorted lookups.  A block takes
// the next tile ticket (kSumTile = 256 lookups); wave w owns the kSumRows =
// 16 lookups [16w, 16w + 16) of the tile, lane j < 16 lookup i0 + j.  (Sixteen
// waves of 16 rows keep more row loads in flight per CU than eight of 32: the
// tiles of the rarest ids, one segment per row, store almost every row they
// load and set the kernel's length.)
//  1. Heads and segment ends come from the neighbouring sorted keys; the
//     block counts its heads and wave 0 numbers the segments by decoupled
//     look-back over earlier tiles (no row load is in flight yet, so the
//     look-back's round trips do not queue behind row traffic).  Heads write
//     the distinct id and the segment's first position.
//  2. Value rows: LPR lanes cover LPR*V consecutive columns of one row
//     (16-byte loads when V = 4), so one load instruction fetches 64/LPR rows;
//     all 16 rows of the wave are requested before any is used, then added in
//     sorted (= lookup) order as they arrive (the compiler waits for each load
//     instruction's rows in turn): row j to the accumulator of lane group
//     j % (64/LPR); a segment that ends at row j is closed by adding the group
//     accumulators pairwise across lanes (one fixed order, the same bits on
//     every lane) unless row j is its only row in the wave.  A segment inside
//     the wave is written with its count; the wave's first segment, if it began
//     before the wave, leaves a double partial in LDS, and so does its last
//     segment if it goes on past the wave.
//  3. A segment that crosses waves inside the tile is summed by the wave where
//     it ends, which walks back to the wave where it started and adds the
//     partials in wave order, and written with its count; all waves do this at
//     once.  What crosses the tile remains: the tile's first segment,
//     begun in an earlier tile (partial in tfirst[tile]), and its last, going
//     on into the next (partial in tlast[tile], and tcross[tile] = its number;
//     -1 when there is none), found by the last wave.
// The last tile writes U (0 when an id was out of range or a wait timed out)
// and seg_start[U] = n.
template <int V, int LPR>
__global__ __launch_bounds__(kSumThreads) void k_seg_sum(
    const uint64_t* __restrict__ s, int64_t n, int pos_bits, int64_t ntiles,
    const float* __restrict__ vals, int64_t width, int64_t* __restrict__ out_keys,
    float* __restrict__ out_vals, int32_t* __restrict__ out_counts, int64_t* d_nunique,
    int32_t* __restrict__ seg_start, double* __restrict__ tfirst, double* __restrict__ tlast,
    int32_t* __restrict__ tcross, uint32_t* words, uint32_t* ticket, uint32_t* status,
    int32_t* __restrict__ bnd, int64_t key_space, const uint32_t* __restrict__ counts) {
    constexpr int RPI = kWave / LPR;
    constexpr int U = kSumRows / RPI;  // load instructions per block of columns
    constexpr int CB = LPR * V;        // columns per block of columns
    static_assert(kSumRows % RPI == 0 && kSumRows <= kWave, "lane groups tile the wave's rows");
    static_assert(CB <= 128, "partials of one block of columns fit the LDS slots");
    __shared__ double pf[kSumWaves][CB];
    __shared__ double pl[kSumWaves][CB];
    __shared__ uint32_t wheads[kSumWaves], wflags[kSumWaves];
    __shared__ int32_t wfirst_end[kSumWaves], wlast_seg[kSumWaves], wlast_head[kSumWaves];
    __shared__ uint32_t wcnt[kSumWaves];
    __shared__ uint32_t s_tile, s_excl, s_ok;
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = lane_id();
    const int sub = lane / LPR, sl = lane % LPR;
    // The status word (an id out of range, a wait that timed out) is loaded
    // while the ticket is taken; nothing is written before it is checked.
    // With per-tile head counts (counts: at most kSumThreads tiles) there is
    // no ticket and no look-back: tile = block, and thread t holds the count
    // of tile t if t comes before this tile, loaded with the keys.
    const uint32_t st0 = *status;
    if (counts == nullptr) {
        if (tid == 0) s_tile = atomicAdd(ticket, 1u);
        __syncthreads();
    }
    const int64_t tile = counts != nullptr ? (int64_t)blockIdx.x : (int64_t)s_tile;
    const uint32_t cbefore = (counts != nullptr && tid < tile) ? counts[tid] : 0u;
    const int64_t i0 = tile * kSumTile + (int64_t)w * kSumRows;
    const int cnt = i0 >= n ? 0 : (int)((n - i0) < kSumRows ? (n - i0) : kSumRows);

    // ---- 1. heads, ends, numbering
    const bool in = lane < cnt;
    const int64_t i = in ? i0 + lane : (i0 < n ? i0 : n - 1);
    const uint64_t key = s[i];
    const uint64_t prev = s[i > 0 ? i - 1 : 0];
    const uint64_t next = s[i + 1 < n ? i + 1 : i];
    if (st0 != 0u) {
        if (tile == 0 && tid == 0) *d_nunique = 0;
        return;
    }
    const uint64_t id = key >> pos_bits;
    const bool head = in && (i == 0 || (prev >> pos_bits) != id);
    const bool ends = in && (i + 1 >= n || (next >> pos_bits) != id);
    const uint32_t pos = (uint32_t)(key & ((1ull << pos_bits) - 1ull));
    const uint64_t hm = ballot(head);
    const uint32_t cw = read_lane(wave_incl_scan(cbefore), kWave - 1);
    if (lane == 0) {
        wheads[w] = (uint32_t)popc64(hm);
        wcnt[w] = cw;
    }
    __syncthreads();
    uint32_t tile_heads = 0, before = 0;
#pragma unroll
    for (int ww = 0; ww < kSumWaves; ++ww) {
        if (ww < w) before += wheads[ww];
        tile_heads += wheads[ww];
    }
    uint32_t excl0 = 0;
    bool ok0 = true;
    if (counts != nullptr) {
#pragma unroll
        for (int ww = 0; ww < kSumWaves; ++ww) excl0 += wcnt[ww];
    } else {
        if (w == 0) {
            uint32_t excl = 0;
            const bool ok = tile_exclusive_prefix(words, tile, tile_heads, &excl);
            if (lane == 0) {
                s_excl = excl;
                s_ok = ok ? 1u : 0u;
            }
        }
        __syncthreads();
        excl0 = s_excl;
        ok0 = s_ok != 0u;
    }
    if (!ok0) {
        if (tid == 0) {
            atomicOr(status, kStatusTimeout);
            *d_nunique = 0;
        }
        return;
    }
    const uint64_t upto = lane == 63 ? ~0ull : ((2ull << lane) - 1ull);
    const uint32_t heads_upto = (uint32_t)popc64(hm & upto);
    const int32_t seg = (int32_t)(excl0 + before + heads_upto) - 1;
    const bool starts_here = heads_upto > 0;  // a head at or before lane j in this wave
    int kind = kFlushNone;
    if (in && (ends || lane == cnt - 1))
        kind = (ends && starts_here) ? kFlushOut : (!starts_here ? kFlushFirst : kFlushLast);
    const uint64_t first_m = ballot(kind == kFlushFirst);
    const uint64_t last_m = ballot(kind == kFlushLast);
    const uint64_t ends_m = ballot(ends);
    if (lane == 0) {
        const int fl = first_m ? __builtin_ctzll(first_m) : 0;
        const int ll = last_m ? __builtin_ctzll(last_m) : 0;
        const uint64_t upto_ll = ll == 63 ? ~0ull : ((2ull << ll) - 1ull);
        uint32_t f = 0;
        if (first_m) f |= 1u | (((ends_m >> fl) & 1ull) ? 2u : 0u);
        if (last_m) f |= 4u;
        wflags[w] = f;
        wfirst_end[w] = (int32_t)(i0 + fl);
        wlast_head[w] = (int32_t)(i0 + 63 - __builtin_clzll((hm & upto_ll) | 1ull));
    }
    const int32_t lseg = read_lane(seg, last_m ? __builtin_ctzll(last_m) : 0);
    if (lane == 0) wlast_seg[w] = lseg;
    if (head) {
        out_keys[seg] = (int64_t)id;
        seg_start[seg] = (int32_t)i;
        if (bnd != nullptr) {
            // Row blocks of kRoBits rows whose first row lies in (previous id,
            // id] have exactly seg ids below them.
            const int64_t b0 = i == 0 ? 0 : (int64_t)((prev >> pos_bits) / kRoBits) + 1;
            for (int64_t b = b0; b <= (int64_t)(id / kRoBits); ++b) bnd[b] = seg;
        }
    }
    if (kind == kFlushOut) {
        const int first = 63 - __builtin_clzll(hm & upto);
        out_counts[seg] = lane - first + 1;
    }
    if (tile == ntiles - 1 && tid == 0) {
        const uint32_t u = excl0 + tile_heads;
        *d_nunique = (int64_t)u;
        seg_start[u] = (int32_t)n;
        if (bnd != nullptr) {  // blocks past the last id: all U ids below them
            const int64_t last = (int64_t)(s[n - 1] >> pos_bits);
            for (int64_t b = last / kRoBits + 1; b <= key_space / kRoBits; ++b) bnd[b] = (int32_t)u;
        }
    }

    // ---- 2. and 3., one block of columns at a time
    for (int64_t c0 = 0; c0 < width; c0 += CB) {
        const int64_t col = c0 + (int64_t)sl * V;
        float row[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // Past the wave's last lookup, reload that lookup's row (unused).
            const int j = u * RPI + sub;
            const int src = j < cnt ? j : (cnt > 0 ? cnt - 1 : 0);
            const uint32_t p = (uint32_t)__shfl((int)pos, src, kWave);
            load_row<V>(row[u], vals + (int64_t)p * width, col, width);
        }
        double acc[V];
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] = 0.0;
#pragma unroll
        for (int j = 0; j < kSumRows; ++j) {
            const int k = j < cnt ? read_lane(kind, j) : kFlushNone;
            const bool single = (hm >> j) & 1ull;  // row j is the segment's only row here
            if (k != kFlushNone && single) {
                // The sum of one row is the row itself (0 + x rounds back to x):
                // no double accumulation.  acc holds zeros here, since every
                // segment before row j closed at or before row j - 1.
                if (sub == j % RPI) {
                    if (k == kFlushOut) {
                        store_row_f<V>(out_vals + (int64_t)read_lane(seg, j) * width + col,
                                       row[j / RPI], col, width);
                    } else {
#pragma unroll
                        for (int v = 0; v < V; ++v) {
                            if (k == kFlushFirst)
                                pf[w][sl * V + v] = (double)row[j / RPI][v];
                            else
                                pl[w][sl * V + v] = (double)row[j / RPI][v];
                        }
                    }
                }
                continue;
            }
            if (j < cnt && sub == j % RPI) {
#pragma unroll
                for (int v = 0; v < V; ++v) acc[v] += (double)row[j / RPI][v];
            }
            if (k != kFlushNone) {
                int owner = j % RPI;
                if (!single) {
                    owner = 0;
#pragma unroll
                    for (int o = LPR; o < kWave; o <<= 1)
#pragma unroll
                        for (int v = 0; v < V; ++v) acc[v] += __shfl_xor(acc[v], o, kWave);
                }
                if (sub == owner) {
                    if (k == kFlushOut) {
                        store_row<V>(out_vals + (int64_t)read_lane(seg, j) * width + col, acc,
                                     col, width);
                    } else {
#pragma unroll
                        for (int v = 0; v < V; ++v) {
                            if (k == kFlushFirst)
                                pf[w][sl * V + v] = acc[v];
                            else
                                pl[w][sl * V + v] = acc[v];
                        }
                    }
                }
#pragma unroll
                for (int v = 0; v < V; ++v) acc[v] = 0.0;
            }
        }
        __syncthreads();
        // Segments that cross waves, each closed by one wave, all waves at
        // once; lane l holds columns l and l + 64 of this block of columns.
        // Wave w's flags: 1 = its first segment began in an earlier wave
        // (partial pf[w]), 2 = that segment ends in wave w, 4 = a segment
        // starts in wave w and goes on past it (partial pl[w]).  A segment is
        // summed as pl[start] (0 if it began before the tile) + pf of every
        // later wave up to its end, in wave order: one fixed order.
        const uint32_t fw = wflags[w];
        // From wave e back over pass-through waves (flag 1 only) to the wave
        // where the segment reaching e started (-1: before the tile).
        auto walk_back = [&](int e, double (&carry)[2]) -> int {
            int j = e;
            while (j >= 0 && (wflags[j] & 4u) == 0u) --j;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = lane + h * kWave;
                carry[h] = (j >= 0 && c < CB) ? pl[j][c] : 0.0;
            }
            for (int ww = j + 1; ww <= e; ++ww)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int c = lane + h * kWave;
                    if (c < CB) carry[h] += pf[ww][c];
                }
            return j;
        };
        if ((fw & 3u) == 3u) {  // the segment that ends in wave w began earlier
            double carry[2];
            const int j = walk_back(w - 1, carry);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int c = lane + h * kWave;
                if (c < CB) carry[h] += pf[w][c];
            }
            if (j >= 0) {
                const int32_t seg0 = wlast_seg[j];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int64_t c = c0 + lane + h * kWave;
                    if (lane + h * kWave < CB && c < width)
                        out_vals[(int64_t)seg0 * width + c] = (float)carry[h];
                }
                if (lane == 0 && c0 == 0) out_counts[seg0] = wfirst_end[w] - wlast_head[j] + 1;
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int64_t c = c0 + lane + h * kWave;
                    if (lane + h * kWave < CB && c < width) tfirst[tile * width + c] = carry[h];
                }
            }
        }
        if (w == kSumWaves - 1) {  // what goes on past the tile
            const bool open = (fw & 4u) != 0u || (fw & 3u) == 1u;
            int32_t cross = -1;
            if (open) {
                double carry[2];
                const int j = walk_back(w, carry);
                double* dst = j >= 0 ? tlast : tfirst;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int64_t c = c0 + lane + h * kWave;
                    if (lane + h * kWave < CB && c < width) dst[tile * width + c] = carry[h];
                }
                if (j >= 0) cross = wlast_seg[j];
            }
            if (lane == 0 && c0 == 0) tcross[tile] = cross;
        }
        __syncthreads();
    }
}

template <int V>
__global__ __launch_bounds__(kFixWaves2 * kWave) void k_tile_fixup(
    const int32_t* __restrict__ tcross, const int32_t* __restrict__ seg_start,
    const double* __restrict__ tfirst, const double* __restrict__ tlast, int64_t width,
    float* __restrict__ out_vals, int32_t* __restrict__ out_counts, const uint32_t* status) {
    __shared__ double part[kFixRuns][kWave * V];
    tile_fixup_body<V, kFixWaves2>(blockIdx.x, tcross, seg_start, tfirst, tlast, width, out_vals,
                                   out_counts, status, part);
}

// csr_from_lookups after the segment kernel, in one launch: the tile combine
// (one block per segment tile, first in dispatch order: a latency chain), then
// the col_indices blocks, then the row_offsets blocks, which read their ids'
// bounds from the per-block counts the segment kernel wrote (bnd; NULL: they
// search the ids).  The combine runs on 4 waves, one double per lane, so that
// the launch keeps 8 blocks per CU; its additions are the same as above.
template <bool VEC>
__global__ __launch_bounds__(kRoThreads) void k_fix_csr(
    const int32_t* __restrict__ tcross, const int32_t* __restrict__ seg_start,
    const double* __restrict__ tfirst, const double* __restrict__ tlast, int64_t cols,
    float* __restrict__ out_vals, int32_t* __restrict__ out_counts, const uint32_t* status,
    int64_t nfix, const int64_t* __restrict__ keys, const int64_t* d_nnz, int64_t nnz_host,
    int64_t rows, int32_t* __restrict__ row_offsets, int64_t nblk_ci,
    int32_t* __restrict__ col_indices, const int32_t* bnd) {
    __shared__ double part[kFixRuns][kWave];
    const int64_t b = blockIdx.x;
    if (b < nfix) {
        tile_fixup_body<1, kRoThreads / kWave>(b, tcross, seg_start, tfirst, tlast, cols,
                                               out_vals, out_counts, status, part);
        return;
    }
    const int64_t nnz = *d_nnz < nnz_host ? *d_nnz : nnz_host;
    if (b < nfix + nblk_ci) {
        csr_col_block(b - nfix, nblk_ci, nnz, cols, col_indices);
        return;
    }
    csr_row_block<VEC>(b - nfix - nblk_ci, keys, nnz_host, nnz, rows, cols, row_offsets, bnd);
}

// Finite check of the lookup values (SPOPT_VALIDATE), run after the pack
// kernel (which zeroes the status word); block 0 also moves the pack blocks'
// range flags into the status word.
__global__ void k_check_finite(const float* __restrict__ v, int64_t len, const uint32_t* pflag,
                               int npack, uint32_t* status) {
    if (blockIdx.x == 0 && (int)threadIdx.x < npack && pflag[threadIdx.x] != 0u)
        atomicOr(status, kStatusRange);
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

// The canonicalisation of coo_from_lookups, shared with csr_from_lookups:
// `what` names the entry point in errors; bnd (NULL: not wanted) receives the
// per-row-block id counts; with fixup false the tile combine is left to the
// caller's launch.
static int canon_run(const char* what, const int64_t* ids, const float* vals, int64_t n,
                     int64_t width, int64_t key_space, int64_t* out_keys, float* out_vals,
                     int32_t* out_counts, int64_t* d_nunique, void* workspace,
                     size_t workspace_bytes, hipStream_t st, uint32_t flags_arg, int32_t* bnd,
                     bool fixup) {
    CanonLayout L;
    if (n >= ((int64_t)1 << 30)) return fail(SPOPT_EOVERFLOW, "%s: n >= 2^30", what);
    if (!canon_layout(n, width, key_space, &L))
        return fail(SPOPT_EINVAL, "%s: bad n=%lld width=%lld key_space=%lld", what,
                    (long long)n, (long long)width, (long long)key_space);
    if (d_nunique == nullptr) return fail(SPOPT_EINVAL, "%s: d_nunique is NULL", what);
    if (n > 0 && (ids == nullptr || vals == nullptr || out_keys == nullptr ||
                  out_vals == nullptr || out_counts == nullptr))
        return fail(SPOPT_EINVAL, "%s: NULL array", what);
    if (n > 0 && (workspace == nullptr || workspace_bytes < L.total))
        return fail(SPOPT_EWORKSPACE, "%s: workspace %zu bytes, need %zu", what,
                    workspace_bytes, L.total);
    if (n == 0) {
        k_write_i64<<<1, 1, 0, st>>>(d_nunique, 0);
        SPOPT_LAUNCHED();
        return SPOPT_OK;
    }
    if (((uintptr_t)workspace & 255u) != 0)
        return fail(SPOPT_EWORKSPACE, "%s: workspace must be 256-byte aligned", what);
    char* ws = (char*)workspace;
    uint64_t* a = (uint64_t*)(ws + L.off_a);
    uint64_t* b = (uint64_t*)(ws + L.off_b);
    uint32_t* status = (uint32_t*)(ws + L.off_status);
    uint32_t* tickets = (uint32_t*)(ws + L.off_tickets);
    uint32_t* part = (uint32_t*)(ws + L.off_part);
    uint32_t* pflag = (uint32_t*)(ws + L.off_pflag);
    uint32_t* words = (uint32_t*)(ws + L.off_words);
    uint32_t* sumwords = (uint32_t*)(ws + L.off_sumwords);
    int32_t* seg_start = (int32_t*)(ws + L.off_segstart);
    int32_t* tcross = (int32_t*)(ws + L.off_tcross);
    double* tfirst = (double*)(ws + L.off_tfirst);
    double* tlast = (double*)(ws + L.off_tlast);

    // Pack and count digits; the pack kernel also zeroes the status word,
    // tickets and look-back words of the kernels after it.
    // Few radix tiles: the first pass takes per-tile digit counts from the
    // pack kernel instead of looking back.
    const bool counted_sort = L.ntiles <= kMaxCountTiles;
    uint32_t* thist0 = counted_sort ? (uint32_t*)(ws + L.off_thist0) : nullptr;
    k_pack<<<(unsigned)L.npack, kThreads, 0, st>>>(ids, n, key_space, L.pos_bits, L.passes,
                                                   L.digit_bits, L.radix, a, part, pflag,
                                                   (uint4*)(ws + L.off_clear),
                                                   (int64_t)(L.clear_bytes / 16), thist0);
    SPOPT_LAUNCHED();
    const bool validate = (flags_arg & SPOPT_VALIDATE) != 0;
    if (validate) {
        const int64_t len = n * width;
        const int grid = (int)(ceil_div(len, 256) < 4096 ? ceil_div(len, 256) : 4096);
        k_check_finite<<<grid, 256, 0, st>>>(vals, len, pflag, (int)L.npack, status);
        SPOPT_LAUNCHED();
        uint32_t h_status = 0;
        SPOPT_HIP(hipMemcpyAsync(&h_status, status, sizeof(uint32_t), hipMemcpyDeviceToHost, st));
        SPOPT_HIP(hipStreamSynchronize(st));
        if (h_status != 0u) return status_to_code(h_status, what);
    } else if (L.passes == 0) {
        // No radix pass folds the pack blocks' range flags into the status word.
        k_check_finite<<<1, 256, 0, st>>>(vals, 0, pflag, (int)L.npack, status);
        SPOPT_LAUNCHED();
    }
    uint64_t* src = a;
    uint64_t* dst = b;
    for (int p = 0; p < L.passes; ++p) {
        const int rem = L.key_bits - p * L.digit_bits;
        const int nbits = rem < L.digit_bits ? rem : L.digit_bits;
        const int shift = L.pos_bits + p * L.digit_bits;
        uint32_t* pwords = words + (int64_t)p * L.ntiles * L.radix;
        k_onesweep<<<(unsigned)L.ntiles, kSortThreads, 0, st>>>(
            src, dst, n, shift, nbits, L.radix, part + (int64_t)p * L.radix, (int)L.npack,
            L.passes * L.radix, p == 0 ? pflag : nullptr, pwords, tickets + p, status,
            p == 0 ? thist0 : nullptr);
        SPOPT_LAUNCHED();
        uint64_t* t = src;
        src = dst;
        dst = t;
    }
    const uint64_t* sorted = src;

    // Segments and sums, tiles of kSumTile sorted lookups, then the ordered
    // combine of segments that cross tiles.  V floats per lane (16- or 8-byte
    // accesses when the width and the value arrays allow them), over the
    // smallest lane group that covers up to 128 columns (32 lanes at most for 2 or
// 4 floats per lane, within the register budget).
    const uintptr_t al = (uintptr_t)vals | (uintptr_t)out_vals;
    const int V = (width % 4 == 0 && (al & 15u) == 0) ? 4 : (width % 2 == 0 && (al & 7u) == 0) ? 2 : 1;
    const int lpr = width <= 16 * V ? 16 : ((width <= 32 * V || V >= 2) ? 32 : 64);
    // Few tiles: their head counts first, summed by each tile instead of a
    // look-back (the counts take the look-back words' place).
    const bool counted = L.nsum <= kSumThreads;
    if (counted) {
        k_head_count<<<(unsigned)L.nsum, kSumTile, 0, st>>>(sorted, n, L.pos_bits, sumwords);
        SPOPT_LAUNCHED();
    }
    auto sum = [&](auto kernel) {
        kernel<<<(unsigned)L.nsum, kSumThreads, 0, st>>>(
            sorted, n, L.pos_bits, L.nsum, vals, width, out_keys, out_vals, out_counts, d_nunique,
            seg_start, tfirst, tlast, tcross, sumwords, tickets + kMaxPasses,
            status, bnd, key_space, counted ? sumwords : nullptr);
    };
    if (V == 4)
        lpr == 16 ? sum(k_seg_sum<4, 16>) : sum(k_seg_sum<4, 32>);
    else if (V == 2)
        lpr == 16 ? sum(k_seg_sum<2, 16>) : sum(k_seg_sum<2, 32>);
    else
        lpr == 16 ? sum(k_seg_sum<1, 16>) : lpr == 32 ? sum(k_seg_sum<1, 32>)
                                                    : sum(k_seg_sum<1, 64>);
    SPOPT_LAUNCHED();

    if (!fixup) return SPOPT_OK;
    // The combine: V doubles per lane over blocks of 64*V columns.
    const int FV = (width % 4 == 0 && width >= 256 && (al & 15u) == 0) ? 4
                   : (width % 2 == 0 && width >= 128 && (al & 7u) == 0) ? 2 : 1;
    auto fix = [&](auto kernel) {
        kernel<<<(unsigned)L.nsum, kFixWaves2 * kWave, 0, st>>>(tcross, seg_start, tfirst, tlast,
                                                                width, out_vals, out_counts,
                                                                status);
    };
    if (FV == 4)
        fix(k_tile_fixup<4>);
    else if (FV == 2)
        fix(k_tile_fixup<2>);
    else
        fix(k_tile_fixup<1>);
    SPOPT_LAUNCHED();
    return SPOPT_OK;
}

extern "C" int coo_from_lookups(const int64_t* ids, const float* vals, int64_t n, int64_t width,
                                int64_t key_space, int64_t* out_keys, float* out_vals,
                                int32_t* out_counts, int64_t* d_nunique, void* workspace,
                                size_t workspace_bytes, void* stream, uint32_t flags) {
    return canon_run("coo_from_lookups", ids, vals, n, width, key_space, out_keys, out_vals,
                     out_counts, d_nunique, workspace, workspace_bytes, (hipStream_t)stream, flags,
                     nullptr, true);
}

namespace spopt {

int csr_lookups_run(const char* what, const int64_t* ids, const float* vals, int64_t n,
                    int64_t rows, int64_t cols, int64_t* out_keys, float* out_vals,
                    int32_t* out_counts, int64_t* d_nunique, int32_t* row_offsets,
                    int32_t* col_indices, void* workspace, size_t workspace_bytes, hipStream_t st,
                    uint32_t flags, FusedCsr* defer, bool* deferred) {
    if (deferred) *deferred = false;
    if (row_offsets == nullptr || rows < 1 || cols < 1)
        return fail(SPOPT_EINVAL, "%s: NULL row_offsets or bad size", what);
    if (n * cols >= ((int64_t)1 << 31))
        return fail(SPOPT_EOVERFLOW, "%s: %lld entries do not fit int32 offsets", what,
                    (long long)(n * cols));
    CanonLayout L;
    if (!canon_layout(n, cols, rows, &L))
        return fail(SPOPT_EINVAL, "%s: bad n=%lld cols=%lld rows=%lld", what, (long long)n,
                    (long long)cols, (long long)rows);
    const bool fused = (cols & 3) == 0 && (col_indices == nullptr || aligned16(col_indices));
    if (!fused) {
        // Columns not in 16-byte groups: the two calls one after the other.
        int rc = canon_run(what, ids, vals, n, cols, rows, out_keys, out_vals, out_counts,
                           d_nunique, workspace, workspace_bytes, st, flags, nullptr, true);
        if (rc) return rc;
        spopt_coo coo{rows, cols, n, d_nunique, out_keys, out_vals};
        return csr_from_coo(&coo, rows, cols, row_offsets, col_indices, out_vals, nullptr,
                            nullptr, (void*)st, 0u);
    }
    char* ws = (char*)workspace;
    int32_t* bnd = (n > 0 && L.bnd_entries > 0) ? (int32_t*)(ws + L.off_bnd) : nullptr;
    int rc = canon_run(what, ids, vals, n, cols, rows, out_keys, out_vals, out_counts, d_nunique,
                       workspace, workspace_bytes, st, flags, bnd, false);
    if (rc) return rc;
    FusedCsr f;
    f.nfix = n > 0 ? L.nsum : 0;
    f.nblk_ro = rows / kRoBits + 1;
    f.nblk_ci = 0;
    if (col_indices != nullptr) {
        f.nblk_ci = ceil_div(n * cols / 4, kRoThreads);
        if (f.nblk_ci > 1024) f.nblk_ci = 1024;
        if (f.nblk_ci < 1) f.nblk_ci = 1;
    }
    f.tcross = n > 0 ? (const int32_t*)(ws + L.off_tcross) : nullptr;
    f.seg_start = n > 0 ? (const int32_t*)(ws + L.off_segstart) : nullptr;
    f.tfirst = n > 0 ? (const double*)(ws + L.off_tfirst) : nullptr;
    f.tlast = n > 0 ? (const double*)(ws + L.off_tlast) : nullptr;
    f.status = n > 0 ? (const uint32_t*)(ws + L.off_status) : nullptr;
    f.keys = out_keys;
    f.vals = out_vals;
    f.counts = out_counts;
    f.d_n = d_nunique;
    f.n = n;
    f.rows = rows;
    f.cols = cols;
    f.row_offsets = row_offsets;
    f.col_indices = col_indices;
    f.bnd = bnd;
    if (defer != nullptr && deferred != nullptr && (flags & SPOPT_VALIDATE) == 0u &&
        aligned16(row_offsets)) {
        *defer = f;
        *deferred = true;
        return SPOPT_OK;
    }
    auto go = [&](auto kernel) {
        kernel<<<(unsigned)(f.nfix + f.nblk_ci + f.nblk_ro), kRoThreads, 0, st>>>(
            f.tcross, f.seg_start, f.tfirst, f.tlast, cols, out_vals, out_counts, f.status,
            f.nfix, out_keys, d_nunique, n, rows, row_offsets, f.nblk_ci, col_indices, bnd);
    };
    if (aligned16(row_offsets))
        go(k_fix_csr<true>);
    else
        go(k_fix_csr<false>);
    SPOPT_LAUNCHED();
    return SPOPT_OK;
}

}  // namespace spopt

extern "C" int csr_from_lookups(const int64_t* ids, const float* vals, int64_t n, int64_t rows,
                                int64_t cols, int64_t* out_keys, float* out_vals,
                                int32_t* out_counts, int64_t* d_nunique, int32_t* row_offsets,
                                int32_t* col_indices, void* workspace, size_t workspace_bytes,
                                void* stream, uint32_t flags) {
    return csr_lookups_run("csr_from_lookups", ids, vals, n, rows, cols, out_keys, out_vals,
                           out_counts, d_nunique, row_offsets, col_indices, workspace,
                           workspace_bytes, (hipStream_t)stream, flags, nullptr, nullptr);
}
