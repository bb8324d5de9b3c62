/*
 * oracle.h - interface of the CPU oracle (test infrastructure only).
 *
 * Host pointers throughout.  Status codes have the same numeric values as the
 * HIP library's so that a test can compare the two; the oracle defines its own
 * copy and includes nothing from the library.
 */
#ifndef SPARSE_OPT_ORACLE_H
#define SPARSE_OPT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ORC_OK = 0,
    ORC_EINVAL = -1,
    ORC_ERANGE = -2,
    ORC_ENOTCANON = -3,
    ORC_ESHAPE = -4,
    ORC_ENONFINITE = -5,
    ORC_EOVERFLOW = -6,
    ORC_EWORKSPACE = -7,
    ORC_EDEVICE = -8,
    ORC_ENOMEM = -9
};

enum { ORC_MODE_LAZY = 0, ORC_MODE_DORMANCY = 1 };
enum { ORC_WD_L2 = 0, ORC_WD_DECOUPLED = 1 };
enum { ORC_CHECK_FINITE = 1 };

/* weight_decay >= 0; wd_mode ORC_WD_L2 (into the gradient) or
 * ORC_WD_DECOUPLED (beside the Adam move, AdamW). */
typedef struct {
    double lr, beta1, beta2, eps;
    int mode;
    double weight_decay;
    int wd_mode;
} orc_adam_cfg;

typedef struct {
    double lr, momentum, weight_decay;
} orc_sgd_cfg;

/* Raw lookups -> canonical COO: keys strictly ascending, duplicate value rows
 * summed in double in lookup order and rounded once, counts = multiplicity. */
int orc_coo_from_lookups(const int64_t* ids, const float* vals, int64_t n, int64_t width,
                         int64_t key_space, int64_t* out_keys, float* out_vals,
                         int32_t* out_counts, int64_t* out_nunique, int flags);

/* Canonical COO over a dense (dim x width) object -> CSR over rows x cols.
 * width == 1: dim == rows*cols, row = idx / cols, col = idx % cols.
 * width == cols: dim == rows, every entry is a full row. */
int orc_csr_from_coo(const int64_t* idx, const float* vals, int64_t nnz, int64_t dim,
                     int64_t width, int64_t rows, int64_t cols, int32_t* row_offsets,
                     int32_t* col_indices, float* out_vals);

/* CSR -> COO over the flattened view, linear = row * cols + col. */
int orc_csr_to_coo(const int32_t* row_offsets, const int32_t* col_indices, const float* vals,
                   int64_t rows, int64_t cols, int64_t* idx, float* out_vals);

/* One Adam step at global step t (t counts this call) on the touched
 * coordinates; state float, arithmetic double. */
int orc_adam_coo_f32(float* p, float* m, float* v, int32_t* ls, int64_t dim, int64_t width,
                     const int64_t* idx, const float* g, int64_t nnz, int64_t t,
                     const orc_adam_cfg* cfg, int flags);
int orc_adam_csr_f32(float* p, float* m, float* v, int32_t* ls, int64_t rows, int64_t cols,
                     const int32_t* row_offsets, const int32_t* col_indices, const float* g,
                     int64_t t, const orc_adam_cfg* cfg, int flags);
/* Row-granular last_step (one int32 per row, ls[rows]): every non-empty row
 * of the CSR gradient must be full (cols entries), else ORC_ESHAPE.  Each
 * coordinate of a touched row uses the row's gap, and the row's last_step
 * becomes t. */
int orc_adam_rows_csr_f32(float* p, float* m, float* v, int32_t* ls, int64_t rows, int64_t cols,
                          const int32_t* row_offsets, const int32_t* col_indices, const float* g,
                          int64_t t, const orc_adam_cfg* cfg, int flags);
int orc_adam_coo_f64(double* p, double* m, double* v, int32_t* ls, int64_t dim,
                     const int64_t* idx, const double* g, int64_t nnz, int64_t t,
                     const orc_adam_cfg* cfg);

/* Forward gather: out[k, :] = params[idx[k], :] for k < n, duplicates
 * allowed.  ORC_ERANGE for an index outside [0, rows); with ORC_CHECK_FINITE,
 * ORC_ENONFINITE when a gathered row holds a NaN or inf.  Nothing is written
 * on error. */
int orc_read_rows(const float* params, int64_t rows, int64_t cols, const int64_t* idx, int64_t n,
                  float* out, int flags);

/* One SGD step on the touched coordinates (b may be NULL when momentum == 0). */
int orc_sgd_coo_f32(float* p, float* b, int64_t dim, int64_t width, const int64_t* idx,
                    const float* g, int64_t nnz, const orc_sgd_cfg* cfg, int flags);
int orc_sgd_csr_f32(float* p, float* b, int64_t rows, int64_t cols, const int32_t* row_offsets,
                    const int32_t* col_indices, const float* g, const orc_sgd_cfg* cfg,
                    int flags);
int orc_sgd_coo_f64(double* p, double* b, int64_t dim, const int64_t* idx, const double* g,
                    int64_t nnz, const orc_sgd_cfg* cfg);

#ifdef __cplusplus
}
#endif

#endif
