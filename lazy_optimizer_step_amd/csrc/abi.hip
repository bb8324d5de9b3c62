// abi.hip - the optimizer handle, error reporting and the step entry points of
// the C ABI declared in sparse_opt.h.
//
// The handle holds the configuration and the global step t (optirs_gpu
// sparse_optimizer page: bias correction uses the number of step calls so
// far, never a per-coordinate count).  Each step computes, in double, the
// scalars that depend only on t and the hyper-parameters; an Adam handle also
// keeps a device table of beta^k (k < kPowTable) built with the host's pow().
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "common.hpp"

namespace spopt {


static thread_local char g_err[512];

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
}

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int status_to_code(uint32_t bits, const char* what) {
    if (bits & kStatusRange) return fail(SPOPT_ERANGE, "%s: index out of range", what);
    if (bits & (kStatusNotCanon | kStatusTouched))
        return fail(SPOPT_ENOTCANON, "%s: gradient is not in canonical form", what);
    if (bits & kStatusNonFinite) return fail(SPOPT_ENONFINITE, "%s: non-finite gradient", what);
    if (bits & kStatusStep)
        return fail(SPOPT_EINVAL, "%s: a touched coordinate has last_step >= t", what);
    if (bits & kStatusPartial)
        return fail(SPOPT_ESHAPE, "%s: a partial row for a table with one last_step per row",
                    what);
    if (bits & kStatusTimeout)
        return fail(SPOPT_EDEVICE, "%s: a device-side wait timed out", what);
    return fail(SPOPT_EINVAL, "%s: status 0x%x", what, bits);
}

std::mutex& validation_mutex() {
    static std::mutex m;
    return m;
}

// One 4-word status block per device, allocated on first use and kept.
uint32_t* device_status_block() {
    static std::vector<uint32_t*> blocks;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
    if ((size_t)dev >= blocks.size()) blocks.resize((size_t)dev + 1, nullptr);
    if (blocks[(size_t)dev] == nullptr) {
        void* p = nullptr;
        if (hipMalloc(&p, 256) != hipSuccess) return nullptr;
        blocks[(size_t)dev] = (uint32_t*)p;
    }
    return blocks[(size_t)dev];
}

int device_status_check(uint32_t* d_status, hipStream_t s, bool check_touched,
                        const char* what) {
    uint32_t h[4] = {0, 0, 0, 0};
    SPOPT_HIP(hipMemcpyAsync(h, d_status, sizeof h, hipMemcpyDeviceToHost, s));
    SPOPT_HIP(hipStreamSynchronize(s));
    if (h[0] != 0u) return status_to_code(h[0], what);
    if (check_touched && h[1] != h[2])
        return fail(SPOPT_ENOTCANON, "%s: touched-row list has %u rows, row_offsets %u", what,
                    h[2], h[1]);
    return SPOPT_OK;
}

}  // namespace spopt

using namespace spopt;

struct spopt_optimizer {
    int32_t kind;
    spopt_adam_config adam;
    spopt_sgd_config sgd;
    int64_t rows, cols;
    float* p;
    float* m;  // Adam m, or SGD momentum buffer
    float* v;
    int32_t* ls;
    int64_t t;
    double* d_pow;  // device [2 * kPowTable]: beta1^k then beta2^k (Adam only)
};

static int check_adam_config(const spopt_adam_config* c) {
    if (!(c->lr >= 0.0) || !isfinite(c->lr))
        return fail(SPOPT_EINVAL, "adam config: lr must be finite and >= 0");
    if (!(c->beta1 >= 0.0 && c->beta1 < 1.0) || !(c->beta2 >= 0.0 && c->beta2 < 1.0))
        return fail(SPOPT_EINVAL, "adam config: beta1 and beta2 must lie in [0, 1)");
    if (!(c->eps > 0.0) || !isfinite(c->eps))
        return fail(SPOPT_EINVAL, "adam config: eps must be finite and > 0");
    if (c->mode != SPOPT_MODE_LAZY && c->mode != SPOPT_MODE_DORMANCY)
        return fail(SPOPT_EINVAL, "adam config: unknown mode %d", c->mode);
    if (!(c->weight_decay >= 0.0) || !isfinite(c->weight_decay))
        return fail(SPOPT_EINVAL, "adam config: weight_decay must be finite and >= 0");
    if (c->weight_decay_mode != SPOPT_WD_L2 && c->weight_decay_mode != SPOPT_WD_DECOUPLED)
        return fail(SPOPT_EINVAL, "adam config: unknown weight_decay_mode %d",
                    c->weight_decay_mode);
    if (c->last_step_per_row != 0 && c->last_step_per_row != 1)
        return fail(SPOPT_EINVAL, "adam config: last_step_per_row must be 0 or 1");
    return SPOPT_OK;
}

static int check_sgd_config(const spopt_sgd_config* c) {
    if (!(c->lr >= 0.0) || !isfinite(c->lr))
        return fail(SPOPT_EINVAL, "sgd config: lr must be finite and >= 0");
    if (!(c->momentum >= 0.0 && c->momentum < 1.0))
        return fail(SPOPT_EINVAL, "sgd config: momentum must lie in [0, 1)");
    if (!(c->weight_decay >= 0.0) || !isfinite(c->weight_decay))
        return fail(SPOPT_EINVAL, "sgd config: weight_decay must be finite and >= 0");
    return SPOPT_OK;
}

extern "C" const char* sparse_opt_last_error(void) { return g_err; }

extern "C" int sparse_opt_host_alloc(size_t bytes, void** host_ptr, void** device_ptr) {
    if (host_ptr == nullptr || device_ptr == nullptr || bytes == 0)
        return fail(SPOPT_EINVAL, "host_alloc: NULL output or zero size");
    void* h = nullptr;
    if (hipHostMalloc(&h, bytes, hipHostMallocMapped) != hipSuccess || h == nullptr) {
        (void)hipGetLastError();
        return fail(SPOPT_ENOMEM, "host_alloc: %zu bytes of pinned host memory", bytes);
    }
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, h, 0) != hipSuccess || d == nullptr) {
        (void)hipGetLastError();
        (void)hipHostFree(h);
        return fail(SPOPT_ENOMEM, "host_alloc: no device mapping for the allocation");
    }
    memset(h, 0, bytes);
    *host_ptr = h;
    *device_ptr = d;
    return SPOPT_OK;
}

extern "C" void sparse_opt_host_free(void* host_ptr) {
    if (host_ptr != nullptr) (void)hipHostFree(host_ptr);
}

extern "C" int sparse_opt_host_device_pointer(void* host_ptr, void** device_ptr) {
    if (host_ptr == nullptr || device_ptr == nullptr)
        return fail(SPOPT_EINVAL, "host_device_pointer: NULL argument");
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, host_ptr, 0) != hipSuccess || d == nullptr) {
        (void)hipGetLastError();
        return fail(SPOPT_EINVAL, "host_device_pointer: %p is not mapped pinned host memory",
                    host_ptr);
    }
    *device_ptr = d;
    return SPOPT_OK;
}

extern "C" int sparse_opt_create(spopt_t* out, int32_t kind, const void* config, int64_t rows,
                                 int64_t cols, float* params, float* m_or_momentum, float* v,
                                 int32_t* last_step) {
    if (out == nullptr || config == nullptr || params == nullptr)
        return fail(SPOPT_EINVAL, "create: NULL argument");
    *out = nullptr;
    if (rows < 1 || cols < 1 || rows > INT64_MAX / cols)
        return fail(SPOPT_EINVAL, "create: bad shape %lld x %lld", (long long)rows,
                    (long long)cols);
    spopt_optimizer h{};
    h.kind = kind;
    h.rows = rows;
    h.cols = cols;
    h.p = params;
    h.m = m_or_momentum;
    h.v = v;
    h.ls = last_step;
    h.t = 0;
    if (kind == SPOPT_KIND_ADAM) {
        h.adam = *(const spopt_adam_config*)config;
        int rc = check_adam_config(&h.adam);
        if (rc) return rc;
        if (m_or_momentum == nullptr || v == nullptr || last_step == nullptr)
            return fail(SPOPT_EINVAL, "create: Adam needs m, v and last_step");
    } else if (kind == SPOPT_KIND_SGD) {
        h.sgd = *(const spopt_sgd_config*)config;
        int rc = check_sgd_config(&h.sgd);
        if (rc) return rc;
        if (h.sgd.momentum != 0.0 && m_or_momentum == nullptr)
            return fail(SPOPT_EINVAL, "create: SGD with momentum needs a momentum buffer");
    } else {
        return fail(SPOPT_EINVAL, "create: unknown kind %d", kind);
    }
    h.d_pow = nullptr;
    if (kind == SPOPT_KIND_ADAM) {
        // beta^k for short dormancy gaps, from the host's pow() in double.
        std::vector<double> tab(2 * (size_t)kPowTable);
        for (int k = 0; k < kPowTable; ++k) {
            tab[(size_t)k] = pow(h.adam.beta1, (double)k);
            tab[(size_t)kPowTable + (size_t)k] = pow(h.adam.beta2, (double)k);
        }
        void* d = nullptr;
        SPOPT_HIP(hipMalloc(&d, tab.size() * sizeof(double)));
        if (hipMemcpy(d, tab.data(), tab.size() * sizeof(double), hipMemcpyHostToDevice) !=
            hipSuccess) {
            (void)hipFree(d);
            return fail(SPOPT_EDEVICE, "create: copying the power table failed");
        }
        h.d_pow = (double*)d;
    }
    spopt_optimizer* p = new (std::nothrow) spopt_optimizer(h);
    if (p == nullptr) {
        if (h.d_pow) (void)hipFree(h.d_pow);
        return fail(SPOPT_EINVAL, "create: out of host memory");
    }
    *out = p;
    return SPOPT_OK;
}

extern "C" void sparse_opt_destroy(spopt_t h) {
    if (h == nullptr) return;
    if (h->d_pow) (void)hipFree(h->d_pow);
    delete h;
}

extern "C" int64_t sparse_opt_get_step(spopt_t h) { return h ? h->t : -1; }

extern "C" int sparse_opt_set_step(spopt_t h, int64_t t) {
    if (h == nullptr) return fail(SPOPT_EINVAL, "set_step: NULL handle");
    if (t < 0 || t >= INT32_MAX) return fail(SPOPT_EINVAL, "set_step: t=%lld out of range",
                                             (long long)t);
    h->t = t;
    return SPOPT_OK;
}

// Shape checks of a gradient against the state (host side, no device access).
static bool row_last_step(const spopt_optimizer* h) {
    return h->kind == SPOPT_KIND_ADAM && h->adam.last_step_per_row != 0;
}

static int check_grad_shape(const spopt_optimizer* h, const spopt_grad* g, const char* what) {
    if (g == nullptr) return fail(SPOPT_EINVAL, "%s: NULL gradient", what);
    if (g->format == SPOPT_FORMAT_COO) {
        const spopt_coo& c = g->coo;
        if (c.nnz < 0) return fail(SPOPT_EINVAL, "%s: nnz < 0", what);
        if (c.nnz > 0 && (c.indices == nullptr || c.values == nullptr))
            return fail(SPOPT_EINVAL, "%s: NULL COO arrays", what);
        const bool flat = c.width == 1 && c.dim == h->rows * h->cols;
        const bool full = c.width == h->cols && c.dim == h->rows;
        if (!flat && !full)
            return fail(SPOPT_ESHAPE,
                        "%s: COO dim %lld width %lld matches neither %lld x 1 nor %lld x %lld",
                        what, (long long)c.dim, (long long)c.width,
                        (long long)(h->rows * h->cols), (long long)h->rows, (long long)h->cols);
        if (row_last_step(h) && !full)
            return fail(SPOPT_ESHAPE,
                        "%s: a table with one last_step per row takes full-row gradients only",
                        what);
        return SPOPT_OK;
    }
    if (g->format == SPOPT_FORMAT_CSR) {
        const spopt_csr& c = g->csr;
        if (c.rows != h->rows || c.cols != h->cols)
            return fail(SPOPT_ESHAPE, "%s: CSR shape %lld x %lld != state %lld x %lld", what,
                        (long long)c.rows, (long long)c.cols, (long long)h->rows,
                        (long long)h->cols);
        if (c.row_offsets == nullptr) return fail(SPOPT_EINVAL, "%s: NULL row_offsets", what);
        if (c.touched_rows && c.n_touched < 0) return fail(SPOPT_EINVAL, "%s: n_touched < 0", what);
        return SPOPT_OK;
    }
    return fail(SPOPT_EINVAL, "%s: unknown gradient format %d", what, g->format);
}

static int validate_grad(const spopt_optimizer* h, const spopt_grad* g, const int32_t* ls,
                         int32_t t, hipStream_t s, const char* what) {
    const bool touched = g->format == SPOPT_FORMAT_CSR && g->csr.touched_rows != nullptr;
    const bool per_row = row_last_step(h);
    // last_step of (row, col): per coordinate row*cols + col; per row, row.  A
    // COO's index is a row (width == cols) or a flattened coordinate (width 1).
    LastStepView lv{ls, t, per_row ? 1 : h->cols, per_row ? 0 : 1, per_row ? 1 : 0};
    return validate_on_device(s, touched, what, [&](uint32_t* status) {
        if (g->format == SPOPT_FORMAT_COO) {
            LastStepView cv = lv;
            cv.ls_rs = per_row ? 1 : g->coo.width;
            return launch_check_coo(&g->coo, 1, cv, status, s);
        }
        return launch_check_csr(&g->csr, 1, lv, status, s);
    });
}

// Timing events a caller asked for, per host thread; the update launchers
// attach them to the dispatch of the kernel that updates the table.
static thread_local hipEvent_t t_ev_begin = nullptr;
static thread_local hipEvent_t t_ev_end = nullptr;

namespace spopt {
StepEvents step_events() { return StepEvents{t_ev_begin, t_ev_end}; }
}  // namespace spopt

extern "C" int sparse_opt_set_step_events(void* begin, void* end) {
    if ((begin == nullptr) != (end == nullptr))
        return fail(SPOPT_EINVAL, "sparse_opt_set_step_events: give both events or neither");
    t_ev_begin = (hipEvent_t)begin;
    t_ev_end = (hipEvent_t)end;
    return SPOPT_OK;
}

// Per-step scalars of Adam at step t, in double on the host.
static AdamScalars adam_scalars(const spopt_optimizer* h, int64_t t) {
    const spopt_adam_config& c = h->adam;
    AdamScalars a;
    a.lr = c.lr;
    a.c1 = 1.0 - c.beta1;
    a.c2 = 1.0 - c.beta2;
    a.bc1 = 1.0 - pow(c.beta1, (double)t);
    a.bc2 = 1.0 - pow(c.beta2, (double)t);
    a.eps = c.eps;
    a.beta1 = c.beta1;
    a.beta2 = c.beta2;
    a.l2b1 = log2(c.beta1);
    a.l2b2 = log2(c.beta2);
    a.pow1 = h->d_pow;
    a.pow2 = h->d_pow + kPowTable;
    a.t = (int32_t)t;
    a.wd = c.weight_decay;
    a.lr_wd = c.lr * c.weight_decay;
    return a;
}

static int adam_wd_kind(const spopt_adam_config& c) {
    return c.weight_decay == 0.0 ? kWdNone
           : c.weight_decay_mode == SPOPT_WD_L2 ? kWdL2 : kWdDecoupled;
}

extern "C" int sparse_adam_step(spopt_t h, const spopt_grad* g, void* stream, uint32_t flags) {
    hipStream_t s = (hipStream_t)stream;
    if (h == nullptr) return fail(SPOPT_EINVAL, "sparse_adam_step: NULL handle");
    if (h->kind != SPOPT_KIND_ADAM) return fail(SPOPT_EINVAL, "sparse_adam_step: not an Adam handle");
    int rc = check_grad_shape(h, g, "sparse_adam_step");
    if (rc) return rc;
    const int64_t t = h->t + 1;
    if (t >= INT32_MAX) return fail(SPOPT_EINVAL, "sparse_adam_step: t would reach 2^31");
    if (flags & SPOPT_VALIDATE) {
        rc = validate_grad(h, g, h->ls, (int32_t)t, s, "sparse_adam_step");
        if (rc) return rc;
    }
    const spopt_adam_config& c = h->adam;
    const AdamScalars a = adam_scalars(h, t);
    const int wd_kind = adam_wd_kind(c);
    rc = launch_adam(h->p, h->m, h->v, h->ls, c.last_step_per_row != 0, a, c.mode, wd_kind, g,
                     h->rows, h->cols, s);
    if (rc) return rc;
    h->t = t;
    return SPOPT_OK;
}

extern "C" int sparse_sgd_step(spopt_t h, const spopt_grad* g, void* stream, uint32_t flags) {
    hipStream_t s = (hipStream_t)stream;
    if (h == nullptr) return fail(SPOPT_EINVAL, "sparse_sgd_step: NULL handle");
    if (h->kind != SPOPT_KIND_SGD) return fail(SPOPT_EINVAL, "sparse_sgd_step: not an SGD handle");
    int rc = check_grad_shape(h, g, "sparse_sgd_step");
    if (rc) return rc;
    const int64_t t = h->t + 1;
    if (t >= INT32_MAX) return fail(SPOPT_EINVAL, "sparse_sgd_step: t would reach 2^31");
    if (flags & SPOPT_VALIDATE) {
        rc = validate_grad(h, g, nullptr, 0, s, "sparse_sgd_step");
        if (rc) return rc;
    }
    const spopt_sgd_config& c = h->sgd;
    rc = launch_sgd(h->p, h->m, c.lr, c.momentum, c.weight_decay, g, h->rows, h->cols, s);
    if (rc) return rc;
    h->t = t;
    return SPOPT_OK;
}

extern "C" int sparse_step_from_lookups(spopt_t h, const int64_t* ids, const float* vals,
                                        int64_t n, int64_t* out_keys, float* out_vals,
                                        int32_t* out_counts, int64_t* d_nunique,
                                        int32_t* row_offsets, int32_t* col_indices,
                                        void* workspace, size_t workspace_bytes, void* stream,
                                        uint32_t flags) {
    hipStream_t s = (hipStream_t)stream;
    if (h == nullptr) return fail(SPOPT_EINVAL, "sparse_step_from_lookups: NULL handle");
    if (h->kind != SPOPT_KIND_ADAM && h->kind != SPOPT_KIND_SGD)
        return fail(SPOPT_EINVAL, "sparse_step_from_lookups: unknown handle kind");
    const int64_t t = h->t + 1;
    if (t >= INT32_MAX) return fail(SPOPT_EINVAL, "sparse_step_from_lookups: t would reach 2^31");
    FusedCsr f;
    bool deferred = false;
    int rc = csr_lookups_run("sparse_step_from_lookups", ids, vals, n, h->rows, h->cols, out_keys,
                             out_vals, out_counts, d_nunique, row_offsets, col_indices, workspace,
                             workspace_bytes, s, flags, &f, &deferred);
    if (rc) return rc;
    if (!deferred) {
        // Validated, or a layout the fused launch does not take: the step
        // call on the CSR just built.
        spopt_grad g;
        memset(&g, 0, sizeof(g));
        g.format = SPOPT_FORMAT_CSR;
        g.csr.rows = h->rows;
        g.csr.cols = h->cols;
        g.csr.row_offsets = row_offsets;
        g.csr.col_indices = col_indices;
        g.csr.values = out_vals;
        g.csr.touched_rows = out_keys;
        g.csr.n_touched = n;
        g.csr.d_n_touched = d_nunique;
        return h->kind == SPOPT_KIND_ADAM ? sparse_adam_step(h, &g, stream, flags)
                                          : sparse_sgd_step(h, &g, stream, flags);
    }
    if (h->kind == SPOPT_KIND_ADAM) {
        const spopt_adam_config& c = h->adam;
        rc = launch_adam_fused(h->p, h->m, h->v, h->ls, c.last_step_per_row != 0,
                               adam_scalars(h, t), c.mode, adam_wd_kind(c), f, s);
    } else {
        const spopt_sgd_config& c = h->sgd;
        rc = launch_sgd_fused(h->p, h->m, c.lr, c.momentum, c.weight_decay, f, s);
    }
    if (rc) return rc;
    h->t = t;
    return SPOPT_OK;
}

// ---- the step from raw lookups without a workspace argument ---------------

// The canonicalisation workspace of sparse_step_from_lookups_noalloc: a
// file-scope device array, one copy on every GPU the library runs on, held
// until the process ends.  Host code never uses this name as an address: the
// device address of each GPU's copy is looked up once, with that GPU current,
// and kept (scratch_address).
constexpr size_t kNoAllocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

static int scratch_address(void** out) {
    static std::mutex mu;
    static std::vector<void*> addr;
    int dev = -1;
    SPOPT_HIP(hipGetDevice(&dev));
    if (dev < 0) return fail(SPOPT_EDEVICE, "sparse_step_from_lookups_noalloc: no current device");
    std::lock_guard<std::mutex> guard(mu);
    if ((size_t)dev >= addr.size()) addr.resize((size_t)dev + 1, nullptr);
    if (addr[(size_t)dev] == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(SPOPT_EDEVICE,
                        "sparse_step_from_lookups_noalloc: device address of the scratch array: %s",
                        hipGetErrorString(e));
        addr[(size_t)dev] = p;
    }
    *out = addr[(size_t)dev];
    return SPOPT_OK;
}

extern "C" int sparse_step_from_lookups_noalloc(spopt_t h, const int64_t* ids, const float* vals,
                                                int64_t n, int64_t* out_keys, float* out_vals,
                                                int32_t* out_counts, int64_t* d_nunique,
                                                int32_t* row_offsets, int32_t* col_indices,
                                                void* stream, uint32_t flags) {
    const char* what = "sparse_step_from_lookups_noalloc";
    if (h == nullptr) return fail(SPOPT_EINVAL, "%s: NULL handle", what);
    if (flags & SPOPT_VALIDATE)
        return fail(SPOPT_EINVAL, "%s: trusted calls only (validation allocates a status block)",
                    what);
    size_t need = 0;
    if (sparse_opt_workspace_size(n, h->cols, h->rows, &need) != SPOPT_OK)
        return fail(SPOPT_EINVAL, "%s: bad n=%lld for a %lld x %lld table", what, (long long)n,
                    (long long)h->rows, (long long)h->cols);
    if (need > kNoAllocScratchBytes)
        return fail(SPOPT_EWORKSPACE,
                    "%s: %lld lookups on a %lld x %lld table need %zu bytes of scratch; the "
                    "fixed scratch holds %zu (use sparse_step_from_lookups with a workspace)",
                    what, (long long)n, (long long)h->rows, (long long)h->cols, need,
                    kNoAllocScratchBytes);
    void* ws = nullptr;
    const int rc = scratch_address(&ws);
    if (rc) return rc;
    return sparse_step_from_lookups(h, ids, vals, n, out_keys, out_vals, out_counts, d_nunique,
                                    row_offsets, col_indices, ws, kNoAllocScratchBytes, stream,
                                    flags);
}
