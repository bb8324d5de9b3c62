// csr.hip - COO <-> CSR on the GPU and the canonical-form checks.
//
// Follows the optirs_gpu sparse_optimizer page, section "Sparse gradient
// representations": a CsrGradient of shape (r, c) and a CooGradient over
// dim = r*c correspond through linear index row*c + col (CsrGradient::to_coo
// and ::from_coo), columns strictly ascending within every row.
//
// row_offsets is built without a global scan: a block owns a run of
// consecutive entries of row_offsets, finds the range of COO entries that fall
// into its rows, counts entries per row in LDS and scans the counts locally
// (the full-row blocks are in csr_full.hpp).  For scalar entries (width 1)
// the kernel that writes the column of every entry also writes the first
// row_offsets entry of every block (the number of entries in the rows below
// it: entry k writes it for the blocks whose first row lies after the row of
// entry k - 1 and at or before its own), so the row blocks read their range
// instead of searching for it; a full-row COO's blocks search its row ids
// once each.
#include "common.hpp"
#include "csr_full.hpp"

namespace spopt {

constexpr int kRoRows = 4096;  // row_offsets entries per block
constexpr int kRoPer = kRoRows / kRoThreads;
constexpr int kRoBatch = 8;    // index loads in flight per thread while counting

// bounds_in_place: row_offsets[r0] and row_offsets[r1] (r1 <= rows) already
// hold the block's entry range, written by k_scalar_cols; the block writes
// row_offsets[r0] again with the same value.
__global__ __launch_bounds__(kRoThreads) void k_row_offsets(
    const int64_t* __restrict__ idx, const int64_t* d_nnz, int64_t nnz_host, int64_t rows,
    int64_t cols, int64_t width, int32_t* __restrict__ row_offsets, int bounds_in_place,
    FastDiv by_cols) {
    __shared__ uint32_t red[kRoThreads / kWave][4];
    __shared__ uint32_t cnt[kRoRows];
    __shared__ uint32_t wt[kRoThreads / kWave];
    const int64_t nnz = d_nnz ? (*d_nnz < nnz_host ? *d_nnz : nnz_host) : nnz_host;
    const int64_t r0 = (int64_t)blockIdx.x * kRoRows;
    const int64_t r1 = (r0 + kRoRows < rows + 1) ? r0 + kRoRows : rows + 1;
    const int64_t scale = (width == 1) ? cols : 1;  // entries of row r have keys < (r+1)*scale
    for (int i = threadIdx.x; i < kRoRows; i += kRoThreads) cnt[i] = 0;
    int64_t ka, kb;
    if (bounds_in_place) {
        // Clamped to [0, nnz], so malformed trusted input never reads outside idx.
        const int64_t a = row_offsets[r0];
        const int64_t b = r1 <= rows ? (int64_t)row_offsets[r1] : nnz;
        ka = a < 0 ? 0 : (a > nnz ? nnz : a);
        kb = b < ka ? ka : (b > nnz ? nnz : b);
        __syncthreads();  // every thread has read row_offsets[r0] before it is written again
    } else {
        const Bounds2 bd = block_lower_bounds2(idx, nnz_host, nnz, r0 * scale, r1 * scale, red);
        ka = bd.b0;
        kb = bd.b1;
    }
    // For canonical input every entry in [ka, kb) lies in rows [r0, r1); the
    // bound test only keeps malformed trusted input inside the LDS array.
    // kRoBatch loads per thread are issued before any is used: a block of the
    // most popular rows holds thousands of entries.
    for (int64_t k0 = ka + threadIdx.x; k0 < kb; k0 += (int64_t)kRoBatch * kRoThreads) {
        int64_t x[kRoBatch];
#pragma unroll
        for (int j = 0; j < kRoBatch; ++j) {
            const int64_t k = k0 + (int64_t)j * kRoThreads;
            x[j] = idx[k < kb ? k : k0];
        }
#pragma unroll
        for (int j = 0; j < kRoBatch; ++j) {
            const bool live = k0 + (int64_t)j * kRoThreads < kb;
            if (scale == 1) {
                const int64_t o = x[j] - r0;
                if (live && (uint64_t)o < (uint64_t)kRoRows) cnt[o] = 1u;
            } else {
                const int64_t o = (x[j] < 0 ? -1 : (int64_t)by_cols.div((uint64_t)x[j]) - r0);
                if (live && (uint64_t)o < (uint64_t)kRoRows) atomicAdd(&cnt[o], 1u);
            }
        }
    }
    __syncthreads();
    uint32_t loc[kRoPer];
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < kRoPer; ++j) {
        loc[j] = cnt[threadIdx.x * kRoPer + j];
        sum += loc[j];
    }
    uint32_t total;
    uint32_t run = block_excl_scan(sum, wt, &total);
#pragma unroll
    for (int j = 0; j < kRoPer; ++j) {
        cnt[threadIdx.x * kRoPer + j] = run;
        run += loc[j];
    }
    __syncthreads();
    const int64_t per_entry = (width == 1) ? 1 : cols;
    // Four offsets per 16-byte store where the block's offsets allow it.  Plain
    // stores, not nontemporal ones: the update that follows scans these offsets.
    if ((((uintptr_t)(row_offsets + r0)) & 15u) == 0 && ((r1 - r0) & 3) == 0) {
        typedef int32_t rx4 __attribute__((ext_vector_type(4)));
        const int nq = (int)((r1 - r0) >> 2);
        for (int q = threadIdx.x; q < nq; q += kRoThreads) {
            const rx4 v = {(int32_t)((ka + (int64_t)cnt[4 * q]) * per_entry),
                           (int32_t)((ka + (int64_t)cnt[4 * q + 1]) * per_entry),
                           (int32_t)((ka + (int64_t)cnt[4 * q + 2]) * per_entry),
                           (int32_t)((ka + (int64_t)cnt[4 * q + 3]) * per_entry)};
            reinterpret_cast<rx4*>(row_offsets + r0)[q] = v;
        }
    } else {
        for (int64_t r = r0 + threadIdx.x; r < r1; r += kRoThreads)
            row_offsets[r] = (int32_t)((ka + (int64_t)cnt[r - r0]) * per_entry);
    }
}

// Full-row COO -> row_offsets and col_indices in one launch: the first nblk_ci
// blocks write col_indices (they search nothing, so their stores overlap the
// row blocks' searches), the rest one row block each.
template <bool VEC>
__global__ __launch_bounds__(kRoThreads) void k_csr_full(
    const int64_t* __restrict__ keys, const int64_t* d_nnz, int64_t nnz_host, int64_t rows,
    int64_t cols, int32_t* __restrict__ row_offsets, int64_t nblk_ci,
    int32_t* __restrict__ col_indices) {
    const int64_t nnz = d_nnz ? (*d_nnz < nnz_host ? *d_nnz : nnz_host) : nnz_host;
    if ((int64_t)blockIdx.x < nblk_ci) {
        csr_col_block(blockIdx.x, nblk_ci, nnz, cols, col_indices);
        return;
    }
    csr_row_block<VEC>((int64_t)blockIdx.x - nblk_ci, keys, nnz_host, nnz, rows, cols,
                       row_offsets, nullptr);
}

// col_indices of full rows: 0..cols-1 repeated for every touched row.
__global__ void k_full_cols(int32_t* __restrict__ ci, const int64_t* d_nnz, int64_t nnz_host,
                            int64_t cols) {
    const int64_t nnz = d_nnz ? (*d_nnz < nnz_host ? *d_nnz : nnz_host) : nnz_host;
    const int64_t total = nnz * cols;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if ((cols & 3) == 0 && aligned16(ci)) {
        for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total / 4; q += stride) {
            const int32_t c = (int32_t)((q * 4) % cols);
            reinterpret_cast<int4*>(ci)[q] = make_int4(c, c + 1, c + 2, c + 3);
        }
    } else {
        for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total; q += stride)
            ci[q] = (int32_t)(q % cols);
    }
}

// Scalar COO over the flattened view: column of every entry, values copied,
// and the first row_offsets entry of every kRoRows-row block: entry k is the
// first entry at or past row b * kRoRows for every block b whose first row
// lies in (row of entry k - 1, row of entry k]; the blocks past the last
// entry's row (all blocks when there is none) hold nnz and are spread over
// every thread of the grid.
__global__ void k_scalar_cols(const int64_t* __restrict__ idx, const float* __restrict__ vin,
                              const int64_t* d_nnz, int64_t nnz_host, int64_t rows, FastDiv by_cols,
                              int32_t* __restrict__ ci, float* __restrict__ vout,
                              int32_t* __restrict__ row_offsets) {
    const int64_t nnz = d_nnz ? (*d_nnz < nnz_host ? *d_nnz : nnz_host) : nnz_host;
    const int64_t nblk = rows / kRoRows;  // blocks 0..nblk start at rows <= rows
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t gstride = (int64_t)gridDim.x * blockDim.x;
    const int64_t xl = nnz > 0 ? idx[nnz - 1] : -1;
    // first block past the last row
    const int64_t after = xl < 0 ? 0 : (int64_t)by_cols.div((uint64_t)xl) / kRoRows + 1;
    for (int64_t b = after + gid; b <= nblk; b += gstride)
        row_offsets[b * kRoRows] = (int32_t)(nnz > 0 ? nnz : 0);
    // Four entries per thread: two 16-byte index loads and one 16-byte column
    // store where the arrays allow it.
    const bool vec = ci != nullptr && ((((uintptr_t)idx) | ((uintptr_t)ci)) & 15u) == 0;
    const int64_t nq = (nnz + 3) / 4;
    for (int64_t q = gid; q < nq; q += gstride) {
        const int64_t k0 = 4 * q;
        int64_t xs[5];
        xs[0] = k0 > 0 ? idx[k0 - 1] : -1;
        if (vec && k0 + 4 <= nnz) {
            const longlong2 a = reinterpret_cast<const longlong2*>(idx + k0)[0];
            const longlong2 b = reinterpret_cast<const longlong2*>(idx + k0)[1];
            xs[1] = a.x; xs[2] = a.y; xs[3] = b.x; xs[4] = b.y;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) xs[j + 1] = k0 + j < nnz ? idx[k0 + j] : -1;
        }
        int32_t cs[4];
        int64_t rowp = xs[0] < 0 ? -1 : (int64_t)by_cols.div((uint64_t)xs[0]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t k = k0 + j;
            const int64_t x = xs[j + 1];
            // Rows as floor(x / cols); -1 below the first entry (or for a negative
            // index, which a trusted caller promises not to pass).
            uint64_t col = 0;
            const int64_t row = x < 0 ? -1 : (int64_t)by_cols.div((uint64_t)x, &col);
            cs[j] = x < 0 ? -1 : (int32_t)col;
            if (k < nnz) {
                if (vout) vout[k] = vin[k];
                int64_t b0 = rowp < 0 ? 0 : rowp / kRoRows + 1;
                int64_t b1 = row < 0 ? -1 : row / kRoRows;
                if (b1 > nblk) b1 = nblk;
                for (int64_t b = b0; b <= b1; ++b) row_offsets[b * kRoRows] = (int32_t)k;
            }
            rowp = row;
        }
        if (ci) {
            if (vec && k0 + 4 <= nnz) {
                reinterpret_cast<int4*>(ci + k0)[0] = make_int4(cs[0], cs[1], cs[2], cs[3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (k0 + j < nnz) ci[k0 + j] = cs[j];
            }
        }
    }
}

__global__ void k_copy_f32(const float* __restrict__ in, float* __restrict__ out,
                           const int64_t* d_nnz, int64_t nnz_host, int64_t width) {
    const int64_t nnz = d_nnz ? (*d_nnz < nnz_host ? *d_nnz : nnz_host) : nnz_host;
    const int64_t total = nnz * width;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    if ((total & 3) == 0 && aligned16(in) && aligned16(out)) {
        for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total / 4; q += stride)
            reinterpret_cast<float4*>(out)[q] = reinterpret_cast<const float4*>(in)[q];
    } else {
        for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total; q += stride)
            out[q] = in[q];
    }
}

__global__ void k_copy_rows(const int64_t* __restrict__ in, int64_t* __restrict__ out,
                            const int64_t* d_nnz, int64_t nnz_host, int64_t* d_count) {
    const int64_t nnz = d_nnz ? (*d_nnz < nnz_host ? *d_nnz : nnz_host) : nnz_host;
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (out && out != in)
        for (int64_t k = g; k < nnz; k += (int64_t)gridDim.x * blockDim.x) out[k] = in[k];
    if (d_count && g == 0) *d_count = nnz;
}

// CSR -> linear COO indices, one wave per 64 rows.
__global__ __launch_bounds__(256) void k_csr_to_coo(const int32_t* __restrict__ ro,
                                                    const int32_t* __restrict__ ci,
                                                    const float* __restrict__ vin, int64_t rows,
                                                    int64_t cols, int64_t* __restrict__ out_idx,
                                                    float* __restrict__ vout) {
    const int lane = lane_id();
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    const int nnz = ro[rows];  // entries stay inside [0, nnz) even for malformed offsets
    for (int64_t tile = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
         tile * kWave < rows; tile += nw) {
        const int64_t r = tile * kWave + lane;
        int a = 0, b = 0;
        if (r < rows) {
            a = ro[r];
            b = ro[r + 1];
        }
        uint64_t mask = ballot(b > a && a >= 0 && b <= nnz);
        while (mask) {
            const int bit = __builtin_ctzll(mask);
            mask &= mask - 1;
            const int st = read_lane(a, bit), en = read_lane(b, bit);
            const int64_t row = tile * kWave + bit;
            for (int j = st + lane; j < en; j += kWave) {
                const int64_t c = ci ? (int64_t)ci[j] : (int64_t)(j - st);
                out_idx[j] = row * cols + c;
                if (vout) vout[j] = vin[j];
            }
        }
    }
}

// ------------------------------------------------------------- checks ---

// COO canonical form, ranges, finiteness, and (for Adam) last_step < t.
__global__ void k_check_coo(const int64_t* __restrict__ idx, const float* __restrict__ vals,
                            const int64_t* d_nnz, int64_t nnz_host, int64_t dim, int64_t width,
                            int check_finite, LastStepView lv, uint32_t* status) {
    const int32_t* __restrict__ ls = lv.ls;
    const int64_t nnz = d_nnz ? (*d_nnz < nnz_host ? *d_nnz : nnz_host) : nnz_host;
    uint32_t bad = 0;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < nnz;
         k += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = idx[k];
        if (i < 0 || i >= dim) {
            bad |= kStatusRange;
            continue;
        }
        if (k > 0 && idx[k - 1] >= i) bad |= kStatusNotCanon;
        for (int64_t c = 0; c < width; ++c) {
            if (check_finite && !finite_f(vals[k * width + c])) bad |= kStatusNonFinite;
            if (ls && ls[i * lv.ls_rs + c * lv.ls_cs] >= lv.t) bad |= kStatusStep;
        }
    }
    if (bad) atomicOr(status, bad);
}

// CSR canonical form (one wave per 64 rows), finiteness, last_step < t, and a
// count of non-empty rows in status[1].
__global__ __launch_bounds__(256) void k_check_csr(const int32_t* __restrict__ ro,
                                                   const int32_t* __restrict__ ci,
                                                   const float* __restrict__ vals, int64_t rows,
                                                   int64_t cols, int check_finite,
                                                   LastStepView lv, uint32_t* status) {
    const int32_t* __restrict__ ls = lv.ls;
    const int lane = lane_id();
    const int64_t nw = ((int64_t)gridDim.x * blockDim.x) >> 6;
    uint32_t bad = 0;
    uint32_t nonempty = 0;
    const int nnz = ro[rows];
    if (blockIdx.x == 0 && threadIdx.x == 0 && (ro[0] != 0 || nnz < 0)) bad |= kStatusNotCanon;
    for (int64_t tile = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 6;
         tile * kWave < rows; tile += nw) {
        const int64_t r = tile * kWave + lane;
        int a = 0, b = 0;
        if (r < rows) {
            a = ro[r];
            b = ro[r + 1];
            if (b < a || a < 0 || b > nnz) {
                bad |= kStatusNotCanon;
                b = a;  // no entry of a malformed row is read
            }
        }
        uint64_t mask = ballot(b > a);
        if (lane == 0) nonempty += (uint32_t)popc64(mask);
        while (mask) {
            const int bit = __builtin_ctzll(mask);
            mask &= mask - 1;
            const int st = read_lane(a, bit), en = read_lane(b, bit);
            const int64_t row = tile * kWave + bit;
            if (ci == nullptr && en - st != cols) bad |= kStatusNotCanon;
            if (lv.full_rows && en - st != cols) bad |= kStatusPartial;
            for (int j = st + lane; j < en; j += kWave) {
                const int64_t c = ci ? (int64_t)ci[j] : (int64_t)(j - st);
                if (c < 0 || c >= cols) {
                    bad |= kStatusRange;
                    continue;
                }
                if (ci && j > st && ci[j - 1] >= c) bad |= kStatusNotCanon;
                if (check_finite && !finite_f(vals[j])) bad |= kStatusNonFinite;
                if (ls && ls[row * lv.ls_rs + c * lv.ls_cs] >= lv.t) bad |= kStatusStep;
            }
        }
    }
    if (bad) atomicOr(status, bad);
    if (lane == 0 && nonempty) atomicAdd(status + 1, nonempty);
}

// Touched-row list: ascending, in range, every listed row non-empty.
__global__ void k_check_touched(const int64_t* __restrict__ tr, const int64_t* d_n,
                                int64_t n_host, const int32_t* __restrict__ ro, int64_t rows,
                                uint32_t* status) {
    const int64_t n = d_n ? (*d_n < n_host ? *d_n : n_host) : n_host;
    uint32_t bad = 0;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < n;
         k += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = tr[k];
        if (r < 0 || r >= rows) {
            bad |= kStatusTouched;
            continue;
        }
        if (k > 0 && tr[k - 1] >= r) bad |= kStatusTouched;
        if (ro[r + 1] <= ro[r]) bad |= kStatusTouched;
    }
    if (bad) atomicOr(status, bad);
    if (blockIdx.x == 0 && threadIdx.x == 0) status[2] = (uint32_t)n;
}

static unsigned grid_for(int64_t work, int64_t per_block, int64_t cap = 4096) {
    int64_t g = ceil_div(work, per_block);
    if (g < 1) g = 1;
    return (unsigned)(g < cap ? g : cap);
}

int launch_check_coo(const spopt_coo* c, int check_finite, const LastStepView& lv,
                     uint32_t* status, hipStream_t s) {
    k_check_coo<<<grid_for(c->nnz, 256), 256, 0, s>>>(c->indices, c->values, c->d_nnz, c->nnz,
                                                      c->dim, c->width, check_finite, lv, status);
    SPOPT_LAUNCHED();
    return SPOPT_OK;
}

int launch_check_csr(const spopt_csr* c, int check_finite, const LastStepView& lv,
                     uint32_t* status, hipStream_t s) {
    k_check_csr<<<grid_for(ceil_div(c->rows, kWave), 4), 256, 0, s>>>(
        c->row_offsets, c->col_indices, c->values, c->rows, c->cols, check_finite, lv, status);
    SPOPT_LAUNCHED();
    if (c->touched_rows) {
        k_check_touched<<<grid_for(c->n_touched, 256), 256, 0, s>>>(
            c->touched_rows, c->d_n_touched, c->n_touched, c->row_offsets, c->rows, status);
        SPOPT_LAUNCHED();
    }
    return SPOPT_OK;
}

}  // namespace spopt

using namespace spopt;

extern "C" int csr_from_coo(const spopt_coo* in, int64_t rows, int64_t cols,
                            int32_t* row_offsets, int32_t* col_indices, float* values,
                            int64_t* touched_rows, int64_t* d_n_touched, void* stream,
                            uint32_t flags) {
    hipStream_t st = (hipStream_t)stream;
    if (in == nullptr || row_offsets == nullptr || rows < 1 || cols < 1 || in->nnz < 0)
        return fail(SPOPT_EINVAL, "csr_from_coo: NULL argument or bad size");
    if (in->nnz > 0 && (in->indices == nullptr || in->values == nullptr))
        return fail(SPOPT_EINVAL, "csr_from_coo: NULL COO arrays");
    const bool full = in->width == cols && in->width > 1;
    if (in->width == 1) {
        if (in->dim != rows * cols)
            return fail(SPOPT_ESHAPE, "csr_from_coo: dim %lld != rows*cols %lld",
                        (long long)in->dim, (long long)(rows * cols));
        if (col_indices == nullptr)
            return fail(SPOPT_EINVAL, "csr_from_coo: col_indices required for scalar entries");
        if (touched_rows != nullptr || d_n_touched != nullptr)
            return fail(SPOPT_EINVAL,
                        "csr_from_coo: touched_rows is produced for full-row COO only");
    } else if (full) {
        if (in->dim != rows)
            return fail(SPOPT_ESHAPE, "csr_from_coo: full-row COO dim %lld != rows %lld",
                        (long long)in->dim, (long long)rows);
    } else {
        return fail(SPOPT_ESHAPE, "csr_from_coo: width %lld is neither 1 nor cols %lld",
                    (long long)in->width, (long long)cols);
    }
    if (in->nnz * in->width >= ((int64_t)1 << 31))
        return fail(SPOPT_EOVERFLOW, "csr_from_coo: %lld entries do not fit int32 offsets",
                    (long long)(in->nnz * in->width));
    if (flags & SPOPT_VALIDATE) {
        const int rc = validate_on_device(st, false, "csr_from_coo", [&](uint32_t* status) {
            return launch_check_coo(in, 0, LastStepView{nullptr, 0, 0, 0, 0}, status, st);
        });
        if (rc) return rc;
    }
    if (full && (cols & 3) == 0 && (col_indices == nullptr || aligned16(col_indices))) {
        // row_offsets and col_indices in one launch.
        const int64_t nblk_ro = ceil_div(rows + 1, kRoBits);
        const int64_t nblk_ci = col_indices ? grid_for(in->nnz * cols / 4, kRoThreads, 1024) : 0;
        if (aligned16(row_offsets))
            k_csr_full<true><<<(unsigned)(nblk_ci + nblk_ro), kRoThreads, 0, st>>>(
                in->indices, in->d_nnz, in->nnz, rows, cols, row_offsets, nblk_ci, col_indices);
        else
            k_csr_full<false><<<(unsigned)(nblk_ci + nblk_ro), kRoThreads, 0, st>>>(
                in->indices, in->d_nnz, in->nnz, rows, cols, row_offsets, nblk_ci, col_indices);
        SPOPT_LAUNCHED();
    } else if (full) {
        k_row_offsets<<<(unsigned)ceil_div(rows + 1, kRoRows), kRoThreads, 0, st>>>(
            in->indices, in->d_nnz, in->nnz, rows, cols, in->width, row_offsets, 0,
            FastDiv::make(1));
        SPOPT_LAUNCHED();
        if (col_indices) {
            k_full_cols<<<grid_for(in->nnz * cols / 4 + 1, 256), 256, 0, st>>>(
                col_indices, in->d_nnz, in->nnz, cols);
            SPOPT_LAUNCHED();
        }
    } else {
        // Scalar entries: columns, values and the row blocks' first offsets,
        // then the row blocks.
        const FastDiv by_cols = FastDiv::make((uint64_t)cols);
        k_scalar_cols<<<grid_for((in->nnz + 3) / 4, 256), 256, 0, st>>>(
            in->indices, in->values, in->d_nnz, in->nnz, rows, by_cols, col_indices,
            values == in->values ? nullptr : values, row_offsets);
        SPOPT_LAUNCHED();
        k_row_offsets<<<(unsigned)ceil_div(rows + 1, kRoRows), kRoThreads, 0, st>>>(
            in->indices, in->d_nnz, in->nnz, rows, cols, in->width, row_offsets, 1, by_cols);
        SPOPT_LAUNCHED();
    }
    if (full) {
        if (values && values != in->values) {
            k_copy_f32<<<grid_for(in->nnz * cols / 4 + 1, 256), 256, 0, st>>>(
                in->values, values, in->d_nnz, in->nnz, cols);
            SPOPT_LAUNCHED();
        }
        if ((touched_rows && touched_rows != in->indices) ||
            (d_n_touched && d_n_touched != in->d_nnz)) {
            k_copy_rows<<<grid_for(in->nnz, 256), 256, 0, st>>>(
                in->indices, touched_rows == in->indices ? nullptr : touched_rows, in->d_nnz,
                in->nnz, d_n_touched == in->d_nnz ? nullptr : d_n_touched);
            SPOPT_LAUNCHED();
        }
    }
    return SPOPT_OK;
}

extern "C" int csr_to_coo(const spopt_csr* in, int64_t* out_indices, float* out_values,
                          void* stream, uint32_t flags) {
    hipStream_t st = (hipStream_t)stream;
    if (in == nullptr || out_indices == nullptr || in->row_offsets == nullptr || in->rows < 1 ||
        in->cols < 1)
        return fail(SPOPT_EINVAL, "csr_to_coo: NULL argument or bad size");
    if (out_values && in->values == nullptr)
        return fail(SPOPT_EINVAL, "csr_to_coo: values requested but CSR has none");
    if (flags & SPOPT_VALIDATE) {
        const int rc = validate_on_device(st, false, "csr_to_coo", [&](uint32_t* status) {
            return launch_check_csr(in, 0, LastStepView{nullptr, 0, 0, 0, 0}, status, st);
        });
        if (rc) return rc;
    }
    k_csr_to_coo<<<grid_for(ceil_div(in->rows, kWave), 4), 256, 0, st>>>(
        in->row_offsets, in->col_indices, in->values, in->rows, in->cols, out_indices,
        out_values);
    SPOPT_LAUNCHED();
    return SPOPT_OK;
}
