/*
 * oracle.c - plain, slow CPU reference of the sparse / lazy optimizer step.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  It shares no code,
 * header, table or helper with the HIP library, and the HIP library never
 * calls it.
 *
 * What it follows (page "optirs_gpu::sparse_optimizer", docs.rs, module page):
 *   - section "Sparse gradient representations": canonical COO (strictly
 *     ascending indices), CSR (strictly ascending columns per row), and the
 *     lossless CSR <-> COO mapping  linear = row * cols + col;
 *   - section "Sparse SGD": params[i] -= lr * grad[i] on touched coordinates,
 *     optional coupled weight decay and momentum applied lazily on them;
 *   - section "LazyAdamMode::Lazy": one decay factor per touch;
 *   - section "LazyAdamMode::DormancyDecay": beta^gap with gap = t - last_step;
 *   - bias correction with the global step t (number of step calls so far).
 * From the DiskSparseAdam README (page 2), only where page 1 is silent:
 *   - "Safe Duplicate Aggregation & Sorted I/O": duplicate indices are summed
 *     and the result is sorted;
 *   - "Explicit Weight Decay Semantics" (Euclidean case): Adam weight decay
 *     "l2" adds wd * w to the gradient, "decoupled" adds it to the descent
 *     direction (AdamW);
 *   - "Validated Inputs": out-of-range indices, wrong shapes and non-finite
 *     gradients are errors;
 *   - active rows computed in float64, storage float32.
 *
 * Every function validates everything before it writes anything, so a
 * rejected call leaves every output and every state array untouched.
 *
 * Arithmetic is double throughout.  The *_f32 entry points load float state,
 * compute in double and round once per stored value; the *_f64 entry points
 * keep state in double and exist so that the pins can check the formulas
 * without float storage in the way.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

/* ------------------------------------------------------------------------ */
/* Canonicalisation of raw lookups                                           */
/* ------------------------------------------------------------------------ */

typedef struct {
    int64_t key;
    int64_t pos;
} key_pos;

/* Order by key, then by lookup position: the same order a stable sort by key
 * produces, so every run of equal keys lists its lookups in input order. */
static int cmp_key_pos(const void* a, const void* b) {
    const key_pos* x = (const key_pos*)a;
    const key_pos* y = (const key_pos*)b;
    if (x->key != y->key) return x->key < y->key ? -1 : 1;
    if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
    return 0;
}

int orc_coo_from_lookups(const int64_t* ids, const float* vals, int64_t n, int64_t width,
                         int64_t key_space, int64_t* out_keys, float* out_vals,
                         int32_t* out_counts, int64_t* out_nunique, int flags) {
    if (n < 0 || width < 1 || key_space < 1 || out_nunique == NULL) return ORC_EINVAL;
    if (n > 0 && (ids == NULL || vals == NULL || out_keys == NULL || out_vals == NULL ||
                  out_counts == NULL))
        return ORC_EINVAL;
    if (n > INT32_MAX) return ORC_EOVERFLOW;
    for (int64_t i = 0; i < n; ++i)
        if (ids[i] < 0 || ids[i] >= key_space) return ORC_ERANGE;
    if (flags & ORC_CHECK_FINITE)
        for (int64_t i = 0; i < n * width; ++i)
            if (!isfinite(vals[i])) return ORC_ENONFINITE;

    key_pos* kp = (key_pos*)malloc((size_t)(n > 0 ? n : 1) * sizeof(key_pos));
    double* acc = (double*)malloc((size_t)width * sizeof(double));
    if (kp == NULL || acc == NULL) {
        free(kp);
        free(acc);
        return ORC_ENOMEM;
    }
    for (int64_t i = 0; i < n; ++i) {
        kp[i].key = ids[i];
        kp[i].pos = i;
    }
    qsort(kp, (size_t)n, sizeof(key_pos), cmp_key_pos);

    int64_t u = 0;
    int64_t i = 0;
    while (i < n) {
        int64_t j = i;
        for (int64_t c = 0; c < width; ++c) acc[c] = 0.0;
        /* one run of equal keys; lookups in input order */
        while (j < n && kp[j].key == kp[i].key) {
            const float* row = vals + kp[j].pos * width;
            for (int64_t c = 0; c < width; ++c) acc[c] += (double)row[c];
            ++j;
        }
        out_keys[u] = kp[i].key;
        out_counts[u] = (int32_t)(j - i);
        for (int64_t c = 0; c < width; ++c) out_vals[u * width + c] = (float)acc[c];
        ++u;
        i = j;
    }
    *out_nunique = u;
    free(kp);
    free(acc);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* COO <-> CSR                                                               */
/* ------------------------------------------------------------------------ */

int orc_csr_from_coo(const int64_t* idx, const float* vals, int64_t nnz, int64_t dim,
                     int64_t width, int64_t rows, int64_t cols, int32_t* row_offsets,
                     int32_t* col_indices, float* out_vals) {
    if (nnz < 0 || rows < 1 || cols < 1 || row_offsets == NULL) return ORC_EINVAL;
    if (nnz > 0 && (idx == NULL || vals == NULL || col_indices == NULL || out_vals == NULL))
        return ORC_EINVAL;
    /* Two accepted COO forms: scalar entries over the flattened rows*cols view,
     * or full-row entries whose indices are row ids. */
    if (width == 1) {
        if (dim != rows * cols) return ORC_ESHAPE;
    } else if (width == cols) {
        if (dim != rows) return ORC_ESHAPE;
    } else {
        return ORC_ESHAPE;
    }
    int64_t total = nnz * width;
    if (total > INT32_MAX) return ORC_EOVERFLOW;
    for (int64_t k = 0; k < nnz; ++k) {
        if (idx[k] < 0 || idx[k] >= dim) return ORC_ERANGE;
        if (k > 0 && idx[k] <= idx[k - 1]) return ORC_ENOTCANON;
    }

    for (int64_t r = 0; r <= rows; ++r) row_offsets[r] = 0;
    for (int64_t k = 0; k < nnz; ++k) {
        int64_t row = (width == 1) ? idx[k] / cols : idx[k];
        row_offsets[row + 1] += (int32_t)width;
    }
    for (int64_t r = 0; r < rows; ++r) row_offsets[r + 1] += row_offsets[r];

    /* Entries arrive in ascending linear order, which is row-major order, so
     * they land in CSR order as they come. */
    int64_t e = 0;
    for (int64_t k = 0; k < nnz; ++k) {
        if (width == 1) {
            col_indices[e] = (int32_t)(idx[k] % cols);
            out_vals[e] = vals[k];
            ++e;
        } else {
            for (int64_t c = 0; c < cols; ++c) {
                col_indices[e] = (int32_t)c;
                out_vals[e] = vals[k * width + c];
                ++e;
            }
        }
    }
    return ORC_OK;
}

/* Canonical-form check of a CSR gradient over rows x cols. */
static int check_csr(const int32_t* row_offsets, const int32_t* col_indices, int64_t rows,
                     int64_t cols) {
    if (row_offsets[0] != 0) return ORC_ENOTCANON;
    for (int64_t r = 0; r < rows; ++r) {
        int32_t a = row_offsets[r], b = row_offsets[r + 1];
        if (b < a) return ORC_ENOTCANON;
        for (int32_t j = a; j < b; ++j) {
            if (col_indices[j] < 0 || col_indices[j] >= cols) return ORC_ERANGE;
            if (j > a && col_indices[j] <= col_indices[j - 1]) return ORC_ENOTCANON;
        }
    }
    return ORC_OK;
}

int orc_csr_to_coo(const int32_t* row_offsets, const int32_t* col_indices, const float* vals,
                   int64_t rows, int64_t cols, int64_t* idx, float* out_vals) {
    if (rows < 1 || cols < 1 || row_offsets == NULL) return ORC_EINVAL;
    int64_t nnz = row_offsets[rows];
    if (nnz > 0 && (col_indices == NULL || vals == NULL || idx == NULL || out_vals == NULL))
        return ORC_EINVAL;
    int rc = check_csr(row_offsets, col_indices, rows, cols);
    if (rc != ORC_OK) return rc;
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t j = row_offsets[r]; j < row_offsets[r + 1]; ++j) {
            idx[j] = r * cols + col_indices[j];
            out_vals[j] = vals[j];
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Per-coordinate updates                                                    */
/* ------------------------------------------------------------------------ */

/* Sparse / lazy Adam on one touched coordinate at global step t.
 * Lazy: one decay factor beta per touch.  DormancyDecay: beta^(t - last_step),
 * i.e. what the moments would hold had the dormant steps carried zero
 * gradients.  Bias correction uses the global t; eps is added after the square
 * root of the bias-corrected second moment.
 * Weight decay, on the touched coordinate only (as page 1 applies SGD's
 * coupled decay), with p0 the value before the step:
 *   "l2":        g <- g + wd * p0 before the moments;
 *   "decoupled": p <- p - lr * (m_hat / (sqrt(v_hat) + eps) + wd * p0),
 *                evaluated as the Adam move followed by  - (lr * wd) * p0.
 * With wd == 0 neither term is applied, so the result is the undecayed one
 * bit for bit. */
static void adam_coord(double* p, double* m, double* v, int32_t* ls, double g, int64_t t,
                       const orc_adam_cfg* c) {
    const double p0 = *p;
    double d1 = c->beta1, d2 = c->beta2;
    if (c->mode == ORC_MODE_DORMANCY) {
        double gap = (double)(t - (int64_t)*ls);
        d1 = pow(c->beta1, gap);
        d2 = pow(c->beta2, gap);
    }
    if (c->weight_decay != 0.0 && c->wd_mode == ORC_WD_L2) g = g + c->weight_decay * p0;
    *m = d1 * *m + (1.0 - c->beta1) * g;
    *v = d2 * *v + (1.0 - c->beta2) * (g * g);
    double m_hat = *m / (1.0 - pow(c->beta1, (double)t));
    double v_hat = *v / (1.0 - pow(c->beta2, (double)t));
    *p = p0 - c->lr * m_hat / (sqrt(v_hat) + c->eps);
    if (c->weight_decay != 0.0 && c->wd_mode == ORC_WD_DECOUPLED)
        *p = *p - (c->lr * c->weight_decay) * p0;
    *ls = (int32_t)t;
}

/* Sparse SGD on one touched coordinate: coupled weight decay adds wd * p to
 * the gradient; heavy-ball momentum (no dampening) when momentum != 0. */
static void sgd_coord(double* p, double* b, double g, const orc_sgd_cfg* c) {
    double gg = g + c->weight_decay * *p;
    if (c->momentum != 0.0) {
        *b = c->momentum * *b + gg;
        *p = *p - c->lr * *b;
    } else {
        *p = *p - c->lr * gg;
    }
}

static int check_adam_cfg(const orc_adam_cfg* c) {
    if (c == NULL) return ORC_EINVAL;
    if (!(c->lr >= 0.0) || !(c->beta1 >= 0.0 && c->beta1 < 1.0) ||
        !(c->beta2 >= 0.0 && c->beta2 < 1.0) || !(c->eps > 0.0) || !isfinite(c->lr) ||
        !isfinite(c->eps))
        return ORC_EINVAL;
    if (c->mode != ORC_MODE_LAZY && c->mode != ORC_MODE_DORMANCY) return ORC_EINVAL;
    if (!(c->weight_decay >= 0.0) || !isfinite(c->weight_decay)) return ORC_EINVAL;
    if (c->wd_mode != ORC_WD_L2 && c->wd_mode != ORC_WD_DECOUPLED) return ORC_EINVAL;
    return ORC_OK;
}

static int check_sgd_cfg(const orc_sgd_cfg* c) {
    if (c == NULL) return ORC_EINVAL;
    if (!(c->lr >= 0.0) || !isfinite(c->lr) || !(c->momentum >= 0.0 && c->momentum < 1.0) ||
        !(c->weight_decay >= 0.0) || !isfinite(c->weight_decay))
        return ORC_EINVAL;
    return ORC_OK;
}

/* Touched coordinates of a COO gradient: entry k, column c maps to coordinate
 * idx[k] * width + c of the dense (dim x width) state. */
static int check_coo(const int64_t* idx, const float* g, int64_t nnz, int64_t dim,
                     int64_t width, int flags) {
    if (nnz < 0 || dim < 1 || width < 1) return ORC_EINVAL;
    if (nnz > 0 && (idx == NULL || g == NULL)) return ORC_EINVAL;
    for (int64_t k = 0; k < nnz; ++k) {
        if (idx[k] < 0 || idx[k] >= dim) return ORC_ERANGE;
        if (k > 0 && idx[k] <= idx[k - 1]) return ORC_ENOTCANON;
    }
    if (flags & ORC_CHECK_FINITE)
        for (int64_t i = 0; i < nnz * width; ++i)
            if (!isfinite(g[i])) return ORC_ENONFINITE;
    return ORC_OK;
}

static int check_csr_grad(const int32_t* row_offsets, const int32_t* col_indices,
                          const float* g, int64_t rows, int64_t cols, int flags) {
    if (rows < 1 || cols < 1 || row_offsets == NULL) return ORC_EINVAL;
    int64_t nnz = row_offsets[rows];
    if (nnz > 0 && (col_indices == NULL || g == NULL)) return ORC_EINVAL;
    int rc = check_csr(row_offsets, col_indices, rows, cols);
    if (rc != ORC_OK) return rc;
    if (flags & ORC_CHECK_FINITE)
        for (int64_t i = 0; i < nnz; ++i)
            if (!isfinite(g[i])) return ORC_ENONFINITE;
    return ORC_OK;
}

/* Every touched coordinate must have last_step < t (gap >= 1). */
static int check_step(int64_t t) {
    if (t < 1) return ORC_EINVAL;
    if (t > INT32_MAX) return ORC_EOVERFLOW;
    return ORC_OK;
}

/* ---- Adam, float storage ------------------------------------------------ */

static void adam_f32(float* p, float* m, float* v, int32_t* ls, int64_t i, double g, int64_t t,
                     const orc_adam_cfg* c) {
    double pp = p[i], mm = m[i], vv = v[i];
    adam_coord(&pp, &mm, &vv, &ls[i], g, t, c);
    p[i] = (float)pp;
    m[i] = (float)mm;
    v[i] = (float)vv;
}

int orc_adam_coo_f32(float* p, float* m, float* v, int32_t* ls, int64_t dim, int64_t width,
                     const int64_t* idx, const float* g, int64_t nnz, int64_t t,
                     const orc_adam_cfg* cfg, int flags) {
    int rc;
    if ((rc = check_adam_cfg(cfg)) || (rc = check_step(t)) ||
        (rc = check_coo(idx, g, nnz, dim, width, flags)))
        return rc;
    if (p == NULL || m == NULL || v == NULL || ls == NULL) return ORC_EINVAL;
    for (int64_t k = 0; k < nnz; ++k)
        for (int64_t c = 0; c < width; ++c)
            if (ls[idx[k] * width + c] >= t) return ORC_EINVAL;
    for (int64_t k = 0; k < nnz; ++k)
        for (int64_t c = 0; c < width; ++c)
            adam_f32(p, m, v, ls, idx[k] * width + c, (double)g[k * width + c], t, cfg);
    return ORC_OK;
}

int orc_adam_csr_f32(float* p, float* m, float* v, int32_t* ls, int64_t rows, int64_t cols,
                     const int32_t* row_offsets, const int32_t* col_indices, const float* g,
                     int64_t t, const orc_adam_cfg* cfg, int flags) {
    int rc;
    if ((rc = check_adam_cfg(cfg)) || (rc = check_step(t)) ||
        (rc = check_csr_grad(row_offsets, col_indices, g, rows, cols, flags)))
        return rc;
    if (p == NULL || m == NULL || v == NULL || ls == NULL) return ORC_EINVAL;
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t j = row_offsets[r]; j < row_offsets[r + 1]; ++j)
            if (ls[r * cols + col_indices[j]] >= t) return ORC_EINVAL;
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t j = row_offsets[r]; j < row_offsets[r + 1]; ++j)
            adam_f32(p, m, v, ls, r * cols + col_indices[j], (double)g[j], t, cfg);
    return ORC_OK;
}

/* Row-granular last_step.  The optirs page's SparseAdam ("Lazy Adam") keeps
 * last_step per coordinate; in a table whose gradients always cover whole
 * rows every coordinate of a row carries the same value, so one int32 per row
 * stores the same state, and a full-row step is the per-coordinate step with
 * the row's value broadcast across the row. */
int orc_adam_rows_csr_f32(float* p, float* m, float* v, int32_t* ls, int64_t rows, int64_t cols,
                          const int32_t* row_offsets, const int32_t* col_indices, const float* g,
                          int64_t t, const orc_adam_cfg* cfg, int flags) {
    int rc;
    if ((rc = check_adam_cfg(cfg)) || (rc = check_step(t)) ||
        (rc = check_csr_grad(row_offsets, col_indices, g, rows, cols, flags)))
        return rc;
    if (p == NULL || m == NULL || v == NULL || ls == NULL) return ORC_EINVAL;
    for (int64_t r = 0; r < rows; ++r) {
        int64_t len = (int64_t)row_offsets[r + 1] - row_offsets[r];
        if (len != 0 && len != cols) return ORC_ESHAPE;
        if (len != 0 && ls[r] >= t) return ORC_EINVAL;
    }
    for (int64_t r = 0; r < rows; ++r) {
        if (row_offsets[r + 1] == row_offsets[r]) continue;
        const int32_t before = ls[r];
        for (int32_t j = row_offsets[r]; j < row_offsets[r + 1]; ++j) {
            int64_t i = r * cols + col_indices[j];
            double pp = p[i], mm = m[i], vv = v[i];
            int32_t l = before;
            adam_coord(&pp, &mm, &vv, &l, (double)g[j], t, cfg);
            p[i] = (float)pp;
            m[i] = (float)mm;
            v[i] = (float)vv;
        }
        ls[r] = (int32_t)t;
    }
    return ORC_OK;
}

/* ---- forward gather ------------------------------------------------------ */

/* DiskSparseAdam README, API reference, read_rows(indices): the rows of the
 * current table for the given indices, with the indices validated and
 * corrupted (non-finite) rows refused. */
int orc_read_rows(const float* params, int64_t rows, int64_t cols, const int64_t* idx, int64_t n,
                  float* out, int flags) {
    if (rows < 1 || cols < 1 || n < 0 || params == NULL) return ORC_EINVAL;
    if (n > 0 && (idx == NULL || out == NULL)) return ORC_EINVAL;
    for (int64_t k = 0; k < n; ++k) {
        if (idx[k] < 0 || idx[k] >= rows) return ORC_ERANGE;
        if (flags & ORC_CHECK_FINITE)
            for (int64_t c = 0; c < cols; ++c)
                if (!isfinite(params[idx[k] * cols + c])) return ORC_ENONFINITE;
    }
    for (int64_t k = 0; k < n; ++k)
        memcpy(out + k * cols, params + idx[k] * cols, sizeof(float) * (size_t)cols);
    return ORC_OK;
}

/* ---- Adam, double storage (for the pins) -------------------------------- */

int orc_adam_coo_f64(double* p, double* m, double* v, int32_t* ls, int64_t dim,
                     const int64_t* idx, const double* g, int64_t nnz, int64_t t,
                     const orc_adam_cfg* cfg) {
    int rc;
    if ((rc = check_adam_cfg(cfg)) || (rc = check_step(t))) return rc;
    if (nnz < 0 || dim < 1 || (nnz > 0 && (idx == NULL || g == NULL))) return ORC_EINVAL;
    for (int64_t k = 0; k < nnz; ++k) {
        if (idx[k] < 0 || idx[k] >= dim) return ORC_ERANGE;
        if (k > 0 && idx[k] <= idx[k - 1]) return ORC_ENOTCANON;
        if (ls[idx[k]] >= t) return ORC_EINVAL;
    }
    for (int64_t k = 0; k < nnz; ++k) {
        int64_t i = idx[k];
        adam_coord(&p[i], &m[i], &v[i], &ls[i], g[k], t, cfg);
    }
    return ORC_OK;
}

/* ---- SGD ---------------------------------------------------------------- */

static void sgd_f32(float* p, float* b, int64_t i, double g, const orc_sgd_cfg* c) {
    double pp = p[i], bb = (b != NULL) ? b[i] : 0.0;
    sgd_coord(&pp, &bb, g, c);
    p[i] = (float)pp;
    if (b != NULL && c->momentum != 0.0) b[i] = (float)bb;
}

int orc_sgd_coo_f32(float* p, float* b, int64_t dim, int64_t width, const int64_t* idx,
                    const float* g, int64_t nnz, const orc_sgd_cfg* cfg, int flags) {
    int rc;
    if ((rc = check_sgd_cfg(cfg)) || (rc = check_coo(idx, g, nnz, dim, width, flags))) return rc;
    if (p == NULL || (cfg->momentum != 0.0 && b == NULL)) return ORC_EINVAL;
    for (int64_t k = 0; k < nnz; ++k)
        for (int64_t c = 0; c < width; ++c)
            sgd_f32(p, b, idx[k] * width + c, (double)g[k * width + c], cfg);
    return ORC_OK;
}

int orc_sgd_csr_f32(float* p, float* b, int64_t rows, int64_t cols, const int32_t* row_offsets,
                    const int32_t* col_indices, const float* g, const orc_sgd_cfg* cfg,
                    int flags) {
    int rc;
    if ((rc = check_sgd_cfg(cfg)) ||
        (rc = check_csr_grad(row_offsets, col_indices, g, rows, cols, flags)))
        return rc;
    if (p == NULL || (cfg->momentum != 0.0 && b == NULL)) return ORC_EINVAL;
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t j = row_offsets[r]; j < row_offsets[r + 1]; ++j)
            sgd_f32(p, b, r * cols + col_indices[j], (double)g[j], cfg);
    return ORC_OK;
}

int orc_sgd_coo_f64(double* p, double* b, int64_t dim, const int64_t* idx, const double* g,
                    int64_t nnz, const orc_sgd_cfg* cfg) {
    int rc;
    if ((rc = check_sgd_cfg(cfg))) return rc;
    if (nnz < 0 || dim < 1 || (nnz > 0 && (idx == NULL || g == NULL)) || p == NULL ||
        (cfg->momentum != 0.0 && b == NULL))
        return ORC_EINVAL;
    for (int64_t k = 0; k < nnz; ++k) {
        if (idx[k] < 0 || idx[k] >= dim) return ORC_ERANGE;
        if (k > 0 && idx[k] <= idx[k - 1]) return ORC_ENOTCANON;
    }
    for (int64_t k = 0; k < nnz; ++k) {
        double bb = (b != NULL) ? b[idx[k]] : 0.0;
        sgd_coord(&p[idx[k]], &bb, g[k], cfg);
        if (b != NULL && cfg->momentum != 0.0) b[idx[k]] = bb;
    }
    return ORC_OK;
}
