// update.hip - gather-update-scatter over the touched coordinates only.
//
// The per-coordinate arithmetic follows the optirs_gpu sparse_optimizer page:
//   Adam, sections "LazyAdamMode::Lazy" / "LazyAdamMode::DormancyDecay":
//     d = beta (Lazy) or beta^(t - last_step) (DormancyDecay)
//     m = d1*m + (1-beta1)*g,  v = d2*v + (1-beta2)*g^2
//     p -= lr * (m/(1-beta1^t)) / (sqrt(v/(1-beta2^t)) + eps),  last_step = t
//   with the optional weight decay of the DiskSparseAdam README ("Explicit
//   Weight Decay Semantics", Euclidean case) on the touched coordinate, p0 its
//   value before the step: "l2" g += wd*p0 first; "decoupled" p -= lr*wd*p0
//   after the move (AdamW).
//   SGD, section "Sparse SGD": g' = g + wd*p; with momentum b = mu*b + g',
//     p -= lr*b; without, p -= lr*g'.
// Arithmetic is double with contraction off, state loaded from and rounded
// once back to float32: the same operations in the same order as the CPU
// oracle, so results agree bit for bit except where beta^gap comes from exp2
// (gaps beyond the pow() table) or a duplicate sum rounds differently.  On
// gfx950 a double FMA issues at the rate of an unpacked float FMA, and the
// kernels are bound by HBM, not by the ALUs.  Scalars that depend only on the
// hyper-parameters and t (1 - beta, 1 - beta^t, beta^gap for short gaps) are
// computed on the host in double.
//
// Work mapping: LPR lanes per touched row, 64/LPR rows per wave at a time and
// a batch of ITERS such groups per wave.  A full row (all cols entries
// present) is moved with 16-byte loads and stores of p, m, v, last_step and g
// (nontemporal for the Adam state); a partial row uses one lane per entry.
// Rows come from a touched-row list (CSR) or the keys of a full-row COO;
// without a list the CSR kernel scans row_offsets 64 rows per wave.  The step
// from raw lookups takes its rows from the canonicalisation's segments and
// shares one launch with the tile combine and the CSR blocks (k_step_lookups).
#include <hip/hip_ext.h>

#include "common.hpp"
#include "csr_full.hpp"
#include "seg_combine.hpp"

namespace spopt {

// Nontemporal 16-byte accesses.  An Adam step reads each touched state row once
// and writes it once; with the nontemporal hint those rows do not displace the
// lines that the canonicalisation of the next step (and any other work) reads,
// and their write-back does not fall into that next step.
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t nt_i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_nt(const float* q) {
    const nt_f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4*>(q));
    return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void store_nt(float* q, const float4 x) {
    __builtin_nontemporal_store((nt_f32x4){x.x, x.y, x.z, x.w}, reinterpret_cast<nt_f32x4*>(q));
}
__device__ __forceinline__ void store_nt4(int32_t* q, int32_t x) {
    __builtin_nontemporal_store((nt_i32x4){x, x, x, x}, reinterpret_cast<nt_i32x4*>(q));
}

// Per-coordinate ops.  A vector step is split into phases so that a kernel can
// issue every load of a batch as straight-line code before it computes:
//   load(i, row, r)   p, m, v (and last_step) of 4 coordinates of row `row`,
//   prep(r, x)        loads that depend on them (beta^gap from the table),
//   compute(r, x, g), store(i, row, r).
// One coordinate at a time: rl = row_last(row) before any coordinate of the
// row, scalar(i, rl, g) per coordinate, row_done(row) after them all.  With
// one last_step per row (LSROW) the row's value is read once and written
// once, so every coordinate of the row sees the value from before the step;
// with one per coordinate, row_last and row_done do nothing.
template <int MODE, int WD = kWdNone, bool LSROW = false>
struct AdamOp {
    static constexpr bool kLsRow = LSROW;
    float* __restrict__ p;
    float* __restrict__ m;
    float* __restrict__ v;
    int32_t* __restrict__ ls;
    AdamScalars a;

    struct Vec {
        float4 p, m, v;
        int4 ls;
    };
    struct Aux {
        double d1[4], d2[4];
    };

    // beta^gap: gap 1 -> beta; gaps below kPowTable -> the host's pow() values
    // (t1, t2, fetched in prep); longer gaps -> exp2(gap * log2 beta), skipped
    // when m = v = 0 (never touched), where any finite factor gives zero.
    __device__ __forceinline__ void coord(float& pp, float& mm, float& vv, int32_t last, double t1,
                                          double t2, float g) const {
#pragma clang fp contract(off)
        double d1 = a.beta1, d2 = a.beta2;
        const double p0 = pp, m0 = mm, v0 = vv;
        double gd = g;
        if (WD == kWdL2) gd = gd + a.wd * p0;
        if (MODE == SPOPT_MODE_DORMANCY) {
            const int32_t gap = a.t - last;
            if (gap != 1) {
                if ((uint32_t)gap < (uint32_t)kPowTable) {
                    d1 = t1;
                    d2 = t2;
                } else if (m0 != 0.0 || v0 != 0.0) {
                    d1 = exp2((double)gap * a.l2b1);
                    d2 = exp2((double)gap * a.l2b2);
                }
            }
        }
        const double m1 = d1 * m0 + a.c1 * gd;
        const double v1 = d2 * v0 + a.c2 * (gd * gd);
        const double m_hat = m1 / a.bc1;
        const double v_hat = v1 / a.bc2;
        double p1 = p0 - a.lr * m_hat / (sqrt(v_hat) + a.eps);
        if (WD == kWdDecoupled) p1 = p1 - a.lr_wd * p0;
        pp = (float)p1;
        mm = (float)m1;
        vv = (float)v1;
    }

    __device__ __forceinline__ int table_index(int32_t last) const {
        const int32_t gap = a.t - last;
        return gap < 0 ? 0 : (gap >= kPowTable ? kPowTable - 1 : gap);
    }

    __device__ __forceinline__ void load(int64_t i, int64_t row, Vec& r) const {
        r.p = load_nt(p + i);
        r.m = load_nt(m + i);
        r.v = load_nt(v + i);
        if (MODE == SPOPT_MODE_DORMANCY && LSROW) {
            const int32_t l = ls[row];  // one address per row: a broadcast
            r.ls = make_int4(l, l, l, l);
        } else if (MODE == SPOPT_MODE_DORMANCY) {
            r.ls = *reinterpret_cast<const int4*>(ls + i);
        } else {
            r.ls = make_int4(0, 0, 0, 0);
        }
    }
    __device__ __forceinline__ void prep(const Vec& r, Aux& x) const {
        if (MODE == SPOPT_MODE_DORMANCY && LSROW) {
            const int k = table_index(r.ls.x);
            const double d1 = a.pow1[k], d2 = a.pow2[k];
            x.d1[0] = x.d1[1] = x.d1[2] = x.d1[3] = d1;
            x.d2[0] = x.d2[1] = x.d2[2] = x.d2[3] = d2;
        } else if (MODE == SPOPT_MODE_DORMANCY) {
            const int i0 = table_index(r.ls.x), i1 = table_index(r.ls.y);
            const int i2 = table_index(r.ls.z), i3 = table_index(r.ls.w);
            x.d1[0] = a.pow1[i0]; x.d2[0] = a.pow2[i0];
            x.d1[1] = a.pow1[i1]; x.d2[1] = a.pow2[i1];
            x.d1[2] = a.pow1[i2]; x.d2[2] = a.pow2[i2];
            x.d1[3] = a.pow1[i3]; x.d2[3] = a.pow2[i3];
        }
    }
    __device__ __forceinline__ void compute(Vec& r, const Aux& x, const float4 g) const {
        coord(r.p.x, r.m.x, r.v.x, r.ls.x, x.d1[0], x.d2[0], g.x);
        coord(r.p.y, r.m.y, r.v.y, r.ls.y, x.d1[1], x.d2[1], g.y);
        coord(r.p.z, r.m.z, r.v.z, r.ls.z, x.d1[2], x.d2[2], g.z);
        coord(r.p.w, r.m.w, r.v.w, r.ls.w, x.d1[3], x.d2[3], g.w);
    }
    __device__ __forceinline__ void store(int64_t i, int64_t row, const Vec& r) const {
        store_nt(p + i, r.p);
        store_nt(m + i, r.m);
        store_nt(v + i, r.v);
        if (LSROW)
            ls[row] = a.t;  // every lane of the row stores the same value
        else
            store_nt4(ls + i, a.t);
    }
    __device__ __forceinline__ int32_t row_last(int64_t row) const {
        return LSROW ? ls[row] : 0;
    }
    __device__ __forceinline__ void row_done(int64_t row) const {
        if (LSROW) ls[row] = a.t;
    }
    __device__ __forceinline__ void scalar(int64_t i, int32_t rl, float g) const {
        float pp = p[i], mm = m[i], vv = v[i];
        const int32_t last = (MODE != SPOPT_MODE_DORMANCY) ? 0 : (LSROW ? rl : ls[i]);
        double t1 = 1.0, t2 = 1.0;
        if (MODE == SPOPT_MODE_DORMANCY) {
            const int k = table_index(last);
            t1 = a.pow1[k];
            t2 = a.pow2[k];
        }
        coord(pp, mm, vv, last, t1, t2, g);
        p[i] = pp;
        m[i] = mm;
        v[i] = vv;
        if (!LSROW) ls[i] = a.t;
    }
};

template <bool MOM>
struct SgdOp {
    float* __restrict__ p;
    float* __restrict__ b;
    double lr, mu, wd;

    struct Vec {
        float4 p, b;
    };
    struct Aux {};

    __device__ __forceinline__ void coord(float& pp, float& bb, float g) const {
#pragma clang fp contract(off)
        const double p0 = pp;
        const double gg = (double)g + wd * p0;
        if (MOM) {
            const double b1 = mu * (double)bb + gg;
            pp = (float)(p0 - lr * b1);
            bb = (float)b1;
        } else {
            pp = (float)(p0 - lr * gg);
        }
    }
    static constexpr bool kLsRow = false;
    __device__ __forceinline__ int32_t row_last(int64_t) const { return 0; }
    __device__ __forceinline__ void row_done(int64_t) const {}
    __device__ __forceinline__ void load(int64_t i, int64_t, Vec& r) const {
        r.p = *reinterpret_cast<const float4*>(p + i);
        if (MOM)
            r.b = *reinterpret_cast<const float4*>(b + i);
        else
            r.b = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __device__ __forceinline__ void prep(const Vec&, Aux&) const {}
    __device__ __forceinline__ void compute(Vec& r, const Aux&, const float4 g) const {
        coord(r.p.x, r.b.x, g.x);
        coord(r.p.y, r.b.y, g.y);
        coord(r.p.z, r.b.z, g.z);
        coord(r.p.w, r.b.w, g.w);
    }
    __device__ __forceinline__ void store(int64_t i, int64_t, const Vec& r) const {
        *reinterpret_cast<float4*>(p + i) = r.p;
        if (MOM) *reinterpret_cast<float4*>(b + i) = r.b;
    }
    __device__ __forceinline__ void scalar(int64_t i, int32_t, float g) const {
        float pp = p[i], bb = MOM ? b[i] : 0.f;
        coord(pp, bb, g);
        p[i] = pp;
        if (MOM) b[i] = bb;
    }
};

// Touched rows given as the keys of a full-row COO: row k's values start at k*cols.
struct SrcBlockCoo {
    const int64_t* __restrict__ idx;
    int64_t cols;
    __device__ __forceinline__ void get(int64_t k, int64_t& row, int64_t& st, int64_t& len) const {
        row = idx[k];
        st = k * cols;
        len = cols;
    }
    __device__ __forceinline__ int64_t col(int64_t, int64_t j) const { return j; }
};

// The segments of the lookup canonicalisation, still in the workspace: row
// keys[k], values at k*cols.  A segment that crosses a segment tile is left
// out (len 0): its sum is not complete until the combine, whose block updates
// that row itself.
struct SrcSegs {
    const int64_t* __restrict__ keys;
    const int32_t* __restrict__ seg_start;
    int64_t cols;
    __device__ __forceinline__ void get(int64_t k, int64_t& row, int64_t& st, int64_t& len) const {
        row = keys[k];
        st = k * cols;
        const int32_t a = seg_start[k], b = seg_start[k + 1];
        len = (a / kSumTile == (b - 1) / kSumTile) ? cols : 0;
    }
    __device__ __forceinline__ int64_t col(int64_t, int64_t j) const { return j; }
};

// Touched rows of a CSR gradient.
struct SrcCsrTouched {
    const int64_t* __restrict__ touched;
    const int32_t* __restrict__ ro;
    const int32_t* __restrict__ ci;
    int64_t rows;
    __device__ __forceinline__ void get(int64_t k, int64_t& row, int64_t& st, int64_t& len) const {
        row = touched[k];
        // Selects rather than an early return, so st and len stay in registers
        // (an out-of-range id reads ro[0] and ro[1]: a table has at least one row).
        const bool in = (uint64_t)row < (uint64_t)rows;
        const int64_t r = in ? row : 0;
        const int64_t a = ro[r], b = ro[r + 1], nnz = ro[rows];
        st = in ? a : 0;
        len = (in && a >= 0 && b <= nnz) ? b - a : 0;  // entries stay in [0, nnz)
    }
    __device__ __forceinline__ int64_t col(int64_t st, int64_t j) const {
        return ci ? (int64_t)ci[st + j] : j;
    }
};

// One touched row (id `row`, values g[st, st + len)) by the LPR lanes sl of a
// group: 16-byte vectors when the row is full and aligned, else one lane per
// entry.  With one last_step per row, every lane reads it before any lane of
// the row writes it (the loads of the first pass below, or row_last), and it
// is written once the row is done.
template <class Op, class Src>
__device__ __forceinline__ void update_row(const Op& op, const Src& src, int64_t row, int64_t st,
                                           int64_t len, int64_t cols, const float* __restrict__ g,
                                           bool vec_ok, int sl, int lpr) {
    const int64_t base = row * cols;
    const int32_t rl = op.row_last(row);
    if (vec_ok && len == cols && (st & 3) == 0) {
        const int64_t nvec = cols >> 2;
        for (int64_t c4 = sl; c4 < nvec; c4 += lpr) {
            typename Op::Vec r;
            typename Op::Aux x;
            op.load(base + 4 * c4, row, r);
            if constexpr (Op::kLsRow) r.ls = make_int4(rl, rl, rl, rl);
            const float4 gv = *reinterpret_cast<const float4*>(g + st + 4 * c4);
            op.prep(r, x);
            op.compute(r, x, gv);
            op.store(base + 4 * c4, row, r);
        }
    } else {
        const int64_t n = len < cols ? len : cols;
        for (int64_t j = sl; j < n; j += lpr) {
            const int64_t c = src.col(st, j);
            if ((uint64_t)c < (uint64_t)cols) op.scalar(base + c, rl, g[st + j]);
        }
        op.row_done(row);
    }
}

// The touched rows of block `bid` of `nblk` (the waves of all nblk blocks
// stride over them together).  Each wave takes a batch of RPW*ITERS
// consecutive touched rows.  Lanes 0..RPW*ITERS-1 first fetch one row each
// (id, start of its values, length), so the dependent index loads of the
// whole batch cost one round trip; then every sub-group issues the 16-byte
// loads of all ITERS of its full rows before it computes and stores any of
// them.  Partial rows (and rows whose values are not 16-byte aligned) take a
// scalar loop, one lane per entry.
template <class Op, class Src, int LPR, int ITERS>
__device__ __forceinline__ void update_rows_body(const Op& op, const Src& src,
                                                 const int64_t* d_count, int64_t count_host,
                                                 int64_t rows, int64_t cols,
                                                 const float* __restrict__ g, int vec_ok,
                                                 int64_t bid, int64_t nblk) {
    const int64_t count = d_count ? (*d_count < count_host ? *d_count : count_host) : count_host;
    constexpr int RPW = kWave / LPR;
    constexpr int BATCH = RPW * ITERS;
    static_assert(BATCH <= kWave, "one lane per row of the batch");
    const int lane = lane_id();
    const int sub = lane / LPR, sl = lane % LPR;
    const int64_t gw = (bid * blockDim.x + threadIdx.x) >> 6;
    const int64_t nw = (nblk * blockDim.x) >> 6;
    const int64_t nvec = cols >> 2;
    for (int64_t k0 = gw * BATCH; k0 < count; k0 += nw * BATCH) {
        int64_t prow = -1, pst = 0, plen = 0;
        if (lane < BATCH && k0 + lane < count) src.get(k0 + lane, prow, pst, plen);
        int64_t row[ITERS], st[ITERS], len[ITERS];
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const int from = it * RPW + sub;
            row[it] = __shfl(prow, from, kWave);
            st[it] = __shfl(pst, from, kWave);
            len[it] = __shfl(plen, from, kWave);
            if ((uint64_t)row[it] >= (uint64_t)rows) len[it] = 0;
        }
        if (vec_ok && nvec <= LPR) {
            // One 16-byte vector per lane covers a full row.  The loads of the
            // batch are straight-line code: a lane without a full row loads
            // element 0 instead and drops the result, so no branch separates
            // the loads and all of them are in flight together.
            typename Op::Vec r[ITERS];
            typename Op::Aux x[ITERS];
            float4 gv[ITERS];
            bool act[ITERS];
#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
                act[it] = len[it] == cols && (st[it] & 3) == 0 && sl < nvec;
                const int64_t off = act[it] ? row[it] * cols + 4 * sl : 0;
                const int64_t goff = act[it] ? st[it] + 4 * sl : 0;
                op.load(off, act[it] ? row[it] : 0, r[it]);
                gv[it] = *reinterpret_cast<const float4*>(g + goff);
            }
#pragma unroll
            for (int it = 0; it < ITERS; ++it) op.prep(r[it], x[it]);
#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
                if (act[it]) {
                    op.compute(r[it], x[it], gv[it]);
                    op.store(row[it] * cols + 4 * sl, row[it], r[it]);
                }
            }
            bool full[ITERS];
#pragma unroll
            for (int it = 0; it < ITERS; ++it) full[it] = len[it] == cols && (st[it] & 3) == 0;
#pragma unroll
            for (int it = 0; it < ITERS; ++it) {
                if (full[it] || len[it] <= 0) continue;
                const int64_t n = len[it] < cols ? len[it] : cols;
                const int32_t rl = op.row_last(row[it]);
                for (int64_t j = sl; j < n; j += LPR) {
                    const int64_t c = src.col(st[it], j);
                    if ((uint64_t)c < (uint64_t)cols)
                        op.scalar(row[it] * cols + c, rl, g[st[it] + j]);
                }
                op.row_done(row[it]);
            }
        } else {
#pragma unroll
            for (int it = 0; it < ITERS; ++it)
                if (len[it] > 0)
                    update_row(op, src, row[it], st[it], len[it], cols, g, vec_ok != 0, sl, LPR);
        }
    }
}

template <class Op, class Src, int LPR, int ITERS>
__global__ __launch_bounds__(256) void k_update_rows(Op op, Src src, const int64_t* d_count,
                                                     int64_t count_host, int64_t rows,
                                                     int64_t cols, const float* __restrict__ g,
                                                     int vec_ok) {
    update_rows_body<Op, Src, LPR, ITERS>(op, src, d_count, count_host, rows, cols, g, vec_ok,
                                          blockIdx.x, gridDim.x);
}

// The step from raw lookups after the segment kernel, in one launch of
// 256-thread blocks, none of which waits on another:
//   [0, nfix)            the combine of the segment that crosses out of
//                        segment tile b, if any, then the update of its row
//                        from the combined sums (read back after a barrier);
//   [nfix, nfix + nupd)  the update of every segment that lies within one
//                        tile, as k_update_rows;
//   then the col_indices and row_offsets blocks of the CSR.
// Each coordinate's arithmetic and each sum's order of additions are those
// of the canonicalisation and step calls, so the results are the same bit for
// bit.
template <class Op, int LPR, int ITERS>
__global__ __launch_bounds__(256) void k_step_lookups(Op op, FusedCsr f, int64_t nupd,
                                                      int vec_ok) {
    __shared__ double part[kFixRuns][kWave];
    int64_t b = blockIdx.x;
    if (b < f.nfix) {
        const int32_t seg = tile_fixup_body<1, 256 / kWave>(b, f.tcross, f.seg_start, f.tfirst,
                                                            f.tlast, f.cols, f.vals, f.counts,
                                                            f.status, part);
        if (seg < 0) return;
        __syncthreads();
        if (threadIdx.x < kWave) {
            const int64_t row = f.keys[seg];
            if ((uint64_t)row < (uint64_t)f.rows)
                update_row(op, SrcSegs{f.keys, f.seg_start, f.cols}, row, (int64_t)seg * f.cols,
                           f.cols, f.cols, f.vals, vec_ok != 0, lane_id(), kWave);
        }
        return;
    }
    b -= f.nfix;
    if (b < nupd) {
        update_rows_body<Op, SrcSegs, LPR, ITERS>(op, SrcSegs{f.keys, f.seg_start, f.cols}, f.d_n,
                                                  f.n, f.rows, f.cols, f.vals, vec_ok, b, nupd);
        return;
    }
    b -= nupd;
    const int64_t nnz = *f.d_n < f.n ? *f.d_n : f.n;
    if (b < f.nblk_ci) {
        csr_col_block(b, f.nblk_ci, nnz, f.cols, f.col_indices);
        return;
    }
    csr_row_block<true>(b - f.nblk_ci, f.keys, f.n, nnz, f.rows, f.cols, f.row_offsets, f.bnd);
}

// CSR without a touched-row list: one wave per 64 rows of row_offsets.
template <class Op>
__global__ __launch_bounds__(256) void k_update_csr_scan(Op op, const int32_t* __restrict__ ro,
                                                         const int32_t* __restrict__ ci,
                                                         int64_t rows, int64_t cols,
                                                         const float* __restrict__ g) {
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
            const int64_t base = row * cols;
            const int32_t rl = op.row_last(row);
            for (int j = st + lane; j < en && j - st < cols; j += kWave) {
                const int64_t c = ci ? (int64_t)ci[j] : (int64_t)(j - st);
                if ((uint64_t)c < (uint64_t)cols) op.scalar(base + c, rl, g[j]);
            }
            op.row_done(row);
        }
    }
}

// Scalar COO entries over the flattened state: one thread per entry.
template <class Op>
__global__ __launch_bounds__(256) void k_update_coo_scalar(Op op, const int64_t* __restrict__ idx,
                                                           const int64_t* d_count,
                                                           int64_t count_host, int64_t dim,
                                                           const float* __restrict__ g) {
    const int64_t count = d_count ? (*d_count < count_host ? *d_count : count_host) : count_host;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < count;
         k += (int64_t)gridDim.x * blockDim.x) {
        const int64_t i = idx[k];
        // A table with one last_step per row reaches this kernel only with one
        // column, where row and coordinate coincide.
        if ((uint64_t)i < (uint64_t)dim) {
            op.scalar(i, op.row_last(i), g[k]);
            op.row_done(i);
        }
    }
}

// ---------------------------------------------------------------- launch ---

static int lanes_per_row(int64_t cols) {
    const int64_t nvec = (cols + 3) / 4;
    if (nvec <= 4) return 4;
    if (nvec <= 16) return 16;
    if (nvec <= 32) return 32;
    return 64;
}

// Blocks of a row-update launch: about what the chip holds at once (256 CUs,
// 3-4 of these blocks each); the waves stride over the rows beyond.  More
// blocks only queue empty ones ahead of whatever the launch does next.
constexpr int64_t kUpdateBlocks = 1024;

static unsigned grid_cap(int64_t blocks, int64_t cap = 4096) {
    if (blocks < 1) blocks = 1;
    return (unsigned)(blocks < cap ? blocks : cap);
}

template <class Op>
struct RowBatch {
    static constexpr int kIters = 4;  // full rows per sub-group in flight
};
template <int MODE, int WD, bool LSROW>
struct RowBatch<AdamOp<MODE, WD, LSROW>> {
    static constexpr int kIters = 2;  // Adam holds more state per row in registers
};

// A kernel that updates a table, on 256-thread blocks.  With the calling
// thread's timing events set, they ride on the dispatch itself
// (hipExtLaunchKernel), so they take the kernel's start and end times without
// stream packets of their own.
template <class K, class... A>
static void launch_update_kernel(K kernel, unsigned grid, hipStream_t s, A... args) {
    const StepEvents ev = step_events();
    if (ev.begin != nullptr)
        hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0, s, ev.begin, ev.end, 0u, args...);
    else
        kernel<<<grid, 256, 0, s>>>(args...);
}

// Touched rows one 256-thread block takes per round (4 lanes per row: one
// row per sub-group at a time).
template <class Op>
static int64_t update_rows_per_block(int lpr) {
    return 4 * (kWave / lpr) * (lpr == 4 ? 1 : RowBatch<Op>::kIters);
}

template <class Op, class Src>
static int launch_rows(const Op& op, const Src& src, const int64_t* d_count, int64_t count,
                       int64_t rows, int64_t cols, const float* g, bool vec_ok, hipStream_t s) {
    constexpr int kIters = RowBatch<Op>::kIters;
    const int lpr = lanes_per_row(cols);
    const unsigned grid =
        grid_cap(ceil_div(count, update_rows_per_block<Op>(lpr)), kUpdateBlocks);
    const int v = vec_ok ? 1 : 0;
    switch (lpr) {
        case 4:
            launch_update_kernel(k_update_rows<Op, Src, 4, 1>, grid, s, op, src, d_count, count,
                                 rows, cols, g, v);
            break;
        case 16:
            launch_update_kernel(k_update_rows<Op, Src, 16, kIters>, grid, s, op, src, d_count,
                                 count, rows, cols, g, v);
            break;
        case 32:
            launch_update_kernel(k_update_rows<Op, Src, 32, kIters>, grid, s, op, src, d_count,
                                 count, rows, cols, g, v);
            break;
        default:
            launch_update_kernel(k_update_rows<Op, Src, 64, kIters>, grid, s, op, src, d_count,
                                 count, rows, cols, g, v);
            break;
    }
    SPOPT_LAUNCHED();
    return SPOPT_OK;
}

// Dispatch one gradient to the kernel family that fits it.
template <class Op>
static int launch_update(const Op& op, bool state_aligned, const spopt_grad* gr, int64_t rows,
                         int64_t cols, hipStream_t s) {
    if (gr->format == SPOPT_FORMAT_COO) {
        const spopt_coo& c = gr->coo;
        if (c.nnz == 0) return SPOPT_OK;
        if (c.width == 1) {
            const unsigned grid = grid_cap(ceil_div(c.nnz, 256));
            launch_update_kernel(k_update_coo_scalar<Op>, grid, s, op, c.indices, c.d_nnz, c.nnz,
                                 rows * cols, c.values);
            SPOPT_LAUNCHED();
            return SPOPT_OK;
        }
        const bool vec_ok = state_aligned && (cols & 3) == 0 && aligned16(c.values);
        return launch_rows(op, SrcBlockCoo{c.indices, cols}, c.d_nnz, c.nnz, rows, cols, c.values,
                           vec_ok, s);
    }
    const spopt_csr& c = gr->csr;
    if (c.touched_rows) {
        if (c.n_touched == 0) return SPOPT_OK;
        const bool vec_ok = state_aligned && (cols & 3) == 0 && aligned16(c.values);
        return launch_rows(op, SrcCsrTouched{c.touched_rows, c.row_offsets, c.col_indices, rows},
                           c.d_n_touched, c.n_touched, rows, cols, c.values, vec_ok, s);
    }
    const unsigned grid = grid_cap(ceil_div(ceil_div(rows, kWave), 4));
    launch_update_kernel(k_update_csr_scan<Op>, grid, s, op, c.row_offsets, c.col_indices, rows,
                         cols, c.values);
    SPOPT_LAUNCHED();
    return SPOPT_OK;
}

template <class Op>
static int launch_fused(const Op& op, bool state_aligned, const FusedCsr& f, hipStream_t s) {
    constexpr int kIters = RowBatch<Op>::kIters;
    const int lpr = lanes_per_row(f.cols);
    const int v = state_aligned && aligned16(f.vals) ? 1 : 0;
    const int64_t nupd =
        f.n > 0 ? grid_cap(ceil_div(f.n, update_rows_per_block<Op>(lpr)), kUpdateBlocks) : 0;
    const unsigned grid = (unsigned)(f.nfix + nupd + f.nblk_ci + f.nblk_ro);
    switch (lpr) {
        case 4:
            launch_update_kernel(k_step_lookups<Op, 4, 1>, grid, s, op, f, nupd, v);
            break;
        case 16:
            launch_update_kernel(k_step_lookups<Op, 16, kIters>, grid, s, op, f, nupd, v);
            break;
        case 32:
            launch_update_kernel(k_step_lookups<Op, 32, kIters>, grid, s, op, f, nupd, v);
            break;
        default:
            launch_update_kernel(k_step_lookups<Op, 64, kIters>, grid, s, op, f, nupd, v);
            break;
    }
    SPOPT_LAUNCHED();
    return SPOPT_OK;
}

// Calls go(op, aligned) with the Adam op of the mode, weight decay and
// last_step layout asked for.
template <int MODE, bool LSROW, class Go>
static int with_adam_mode(float* p, float* m, float* v, int32_t* ls, const AdamScalars& a,
                          int wd_kind, bool al, Go&& go) {
    if (wd_kind == kWdL2) return go(AdamOp<MODE, kWdL2, LSROW>{p, m, v, ls, a}, al);
    if (wd_kind == kWdDecoupled) return go(AdamOp<MODE, kWdDecoupled, LSROW>{p, m, v, ls, a}, al);
    return go(AdamOp<MODE, kWdNone, LSROW>{p, m, v, ls, a}, al);
}

template <class Go>
static int with_adam_op(float* p, float* m, float* v, int32_t* ls, bool ls_per_row,
                        const AdamScalars& a, int mode, int wd_kind, Go&& go) {
    // With one last_step per row, only p, m and v are moved 16 bytes at a time.
    const bool al = aligned16(p) && aligned16(m) && aligned16(v) && (ls_per_row || aligned16(ls));
    if (ls_per_row) {
        if (mode == SPOPT_MODE_DORMANCY)
            return with_adam_mode<SPOPT_MODE_DORMANCY, true>(p, m, v, ls, a, wd_kind, al, go);
        return with_adam_mode<SPOPT_MODE_LAZY, true>(p, m, v, ls, a, wd_kind, al, go);
    }
    if (mode == SPOPT_MODE_DORMANCY)
        return with_adam_mode<SPOPT_MODE_DORMANCY, false>(p, m, v, ls, a, wd_kind, al, go);
    return with_adam_mode<SPOPT_MODE_LAZY, false>(p, m, v, ls, a, wd_kind, al, go);
}

template <class Go>
static int with_sgd_op(float* p, float* b, double lr, double mu, double wd, Go&& go) {
    if (mu != 0.0 && b != nullptr) return go(SgdOp<true>{p, b, lr, mu, wd}, aligned16(p) && aligned16(b));
    return go(SgdOp<false>{p, nullptr, lr, 0.0, wd}, aligned16(p));
}

int launch_adam(float* p, float* m, float* v, int32_t* ls, bool ls_per_row, const AdamScalars& a,
                int mode, int wd_kind, const spopt_grad* gr, int64_t rows, int64_t cols,
                hipStream_t s) {
    return with_adam_op(p, m, v, ls, ls_per_row, a, mode, wd_kind, [&](const auto& op, bool al) {
        return launch_update(op, al, gr, rows, cols, s);
    });
}

int launch_adam_fused(float* p, float* m, float* v, int32_t* ls, bool ls_per_row,
                      const AdamScalars& a, int mode, int wd_kind, const FusedCsr& f,
                      hipStream_t s) {
    return with_adam_op(p, m, v, ls, ls_per_row, a, mode, wd_kind,
                        [&](const auto& op, bool al) { return launch_fused(op, al, f, s); });
}

int launch_sgd(float* p, float* b, double lr, double mu, double wd, const spopt_grad* gr,
               int64_t rows, int64_t cols, hipStream_t s) {
    return with_sgd_op(p, b, lr, mu, wd, [&](const auto& op, bool al) {
        return launch_update(op, al, gr, rows, cols, s);
    });
}

int launch_sgd_fused(float* p, float* b, double lr, double mu, double wd, const FusedCsr& f,
                     hipStream_t s) {
    return with_sgd_op(p, b, lr, mu, wd,
                       [&](const auto& op, bool al) { return launch_fused(op, al, f, s); });
}

}  // namespace spopt
