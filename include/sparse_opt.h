/*
 * sparse_opt.h - C ABI of the MI355X (gfx950) sparse / lazy optimizer step.
 *
 * What the library computes (page "optirs_gpu::sparse_optimizer", docs.rs):
 *   - section "Sparse gradient representations": a COO gradient keeps its
 *     indices strictly ascending; a CSR gradient keeps row_offsets, and
 *     strictly ascending col_indices within each row, with the dense shape;
 *     CSR of shape (r, c) and COO over dim = r*c convert losslessly through
 *     linear = row*c + col;
 *   - section "Sparse SGD": params[i] -= lr * grad[i] on touched coordinates
 *     only, with optional coupled weight decay and momentum applied lazily;
 *   - sections "LazyAdamMode::Lazy" and "LazyAdamMode::DormancyDecay": per
 *     coordinate m, v and last_step; Lazy decays once per touch, DormancyDecay
 *     by beta^gap with gap = t - last_step; both bias-correct with the global
 *     step t (the number of step calls so far) and apply
 *     p -= lr * m_hat / (sqrt(v_hat) + eps).
 * Untouched coordinates are never read or written, so they stay bit-identical.
 * From the DiskSparseAdam README, where the optirs page is silent: duplicate
 * lookups are summed and emitted in ascending order ("Safe Duplicate
 * Aggregation & Sorted I/O"); out-of-range indices, wrong shapes and
 * non-finite gradients are errors ("Validated Inputs"; step() method).
 *
 * Conventions for every entry point:
 *   - Pointers named d_* or documented as "device" are HIP device pointers
 *     (e.g. torch tensor data_ptr()); the caller allocates and owns all of
 *     them, including state, outputs and workspace.  The library itself
 *     allocates device memory in two places only: sparse_opt_create makes a
 *     16 KB table of beta1^k and beta2^k (k < 1024, double) for every Adam
 *     handle, freed by sparse_opt_destroy; and the first SPOPT_VALIDATE call
 *     on a device makes a 256-byte status block for that device, kept until
 *     the process ends (validated calls are serialised process-wide around
 *     it).  Step, canonicalisation and conversion calls allocate nothing.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream) on
 *     the calling thread's current device.  All device work is enqueued on
 *     it; calls return before it finishes unless SPOPT_VALIDATE is set, in
 *     which case they synchronise on `stream` once.
 *   - Return value: SPOPT_OK (0) or a negative spopt_status.  No exception
 *     crosses the ABI.  sparse_opt_last_error() gives a message for the
 *     calling thread's most recent failure.
 *   - A call that returns an error has enqueued no kernel that writes an
 *     output or state array, with two documented exceptions: in trusted mode
 *     coo_from_lookups cannot see device-side errors, so it marks its result
 *     empty instead (see there); and sparse_step_from_lookups writes its
 *     canonical outputs before the step's own checks (see there).
 *   - Trusted calls allocate nothing and never synchronise, so they can be
 *     captured into a HIP graph; but a step's scalars (t, 1 - beta^t, ...) are
 *     kernel arguments formed on the host at the call, so a captured step
 *     replays the t it was captured with (and the handle's t advances only at
 *     the capture): capture the canonicalisation alone, or one graph per step.
 *   - Layouts are row-major and contiguous; float arrays whose width is a
 *     multiple of 4 take 16-byte vector loads when their base is 16-byte
 *     aligned (torch allocations are), and a scalar path otherwise.
 */
#ifndef SPARSE_OPT_H
#define SPARSE_OPT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Only the entry points below are exported from the shared library. */
#define SPOPT_API __attribute__((visibility("default")))

/* ---- status codes ------------------------------------------------------- */
typedef enum spopt_status {
    SPOPT_OK = 0,
    SPOPT_EINVAL = -1,      /* bad argument: NULL pointer, size, hyper-parameter, step */
    SPOPT_ERANGE = -2,      /* an index outside its range */
    SPOPT_ENOTCANON = -3,   /* indices not strictly ascending / CSR not canonical */
    SPOPT_ESHAPE = -4,      /* gradient shape does not match the state */
    SPOPT_ENONFINITE = -5,  /* a gradient value is NaN or infinite (SPOPT_VALIDATE) */
    SPOPT_EOVERFLOW = -6,   /* a count does not fit its index type */
    SPOPT_EWORKSPACE = -7,  /* workspace missing or too small */
    SPOPT_EDEVICE = -8,     /* a HIP runtime call failed */
    SPOPT_ENOMEM = -9       /* an allocation the call was asked to make failed */
} spopt_status;

/* ---- flags -------------------------------------------------------------- */
#define SPOPT_TRUSTED 0u   /* no checks beyond bounds guards, no host synchronisation */
#define SPOPT_VALIDATE 1u  /* full input checks on the device, one synchronisation,
                              and a rejected call writes nothing */

/* ---- optimizer kinds and configuration ---------------------------------- */
#define SPOPT_KIND_ADAM 0
#define SPOPT_KIND_SGD 1

#define SPOPT_MODE_LAZY 0      /* LazyAdamMode::Lazy */
#define SPOPT_MODE_DORMANCY 1  /* LazyAdamMode::DormancyDecay */

#define SPOPT_WD_L2 0         /* weight decay added to the gradient (Adam L2) */
#define SPOPT_WD_DECOUPLED 1  /* weight decay beside the Adam move (AdamW) */

/* Sparse / lazy Adam.  lr >= 0, beta1 and beta2 in [0, 1), eps > 0,
 * weight_decay >= 0 (ranges of the DiskSparseAdam API reference; lr >= 0 is
 * this library's own rule).  Doubles: every derived scalar (1 - beta, bias
 * corrections, log2 beta, lr * weight_decay) is formed in double on the host
 * and rounded once.
 * Weight decay (DiskSparseAdam README, "Explicit Weight Decay Semantics", its
 * Euclidean case), applied to touched coordinates only, with p0 the value
 * before the step: SPOPT_WD_L2 adds weight_decay * p0 to the gradient before
 * the moments; SPOPT_WD_DECOUPLED subtracts lr * weight_decay * p0 after the
 * Adam move (AdamW).  weight_decay == 0 is the undecayed step bit for bit. */
typedef struct spopt_adam_config {
    double lr, beta1, beta2, eps;
    int32_t mode; /* SPOPT_MODE_LAZY or SPOPT_MODE_DORMANCY */
    double weight_decay;
    int32_t weight_decay_mode; /* SPOPT_WD_L2 or SPOPT_WD_DECOUPLED */
    /* 0: last_step holds one int32 per coordinate (rows x cols), the form of
     * the optirs_gpu sparse_optimizer page ("Lazy Adam").  1: one int32 per
     * row (rows), for tables whose gradients always cover whole rows: every
     * coordinate of a row then holds the same value, so this stores the same
     * state in fewer bytes.  Such a table takes full-row gradients only: a COO
     * over the flattened view (width 1 with cols > 1) is SPOPT_ESHAPE; a CSR
     * row with some but not all of its columns is SPOPT_ESHAPE under
     * SPOPT_VALIDATE and leaves the table unspecified in trusted mode. */
    int32_t last_step_per_row;
} spopt_adam_config;

/* Sparse SGD.  lr >= 0, momentum in [0, 1), weight_decay >= 0.  Coupled weight
 * decay: g' = g + weight_decay * p.  momentum != 0: b = momentum * b + g',
 * p -= lr * b (heavy ball, no dampening); momentum == 0: p -= lr * g'. */
typedef struct spopt_sgd_config {
    double lr, momentum, weight_decay;
} spopt_sgd_config;

/* ---- gradients ---------------------------------------------------------- */

/* COO gradient over a dense (dim x width) object: entry k covers coordinates
 * indices[k]*width + j for j < width, with values[k*width + j].
 *   width == 1: the optirs_gpu sparse_optimizer page's CooGradient (a 1-D
 *               vector, or the rows*cols flattened view of a table);
 *   width == cols of a table: indices are row ids and every entry is a full
 *               row (the compact form of a CSR whose touched rows are full).
 * indices strictly ascending in [0, dim).
 * The entry count is nnz, or, when d_nnz != NULL, the device value *d_nnz
 * (which must be <= nnz; nnz is then the upper bound used to size launches).
 */
typedef struct spopt_coo {
    int64_t dim;
    int64_t width;
    int64_t nnz;
    const int64_t* d_nnz;   /* device, optional */
    const int64_t* indices; /* device [nnz] */
    const float* values;    /* device [nnz * width] */
} spopt_coo;

/* CSR gradient of shape rows x cols: row r holds entries
 * [row_offsets[r], row_offsets[r+1]) with columns col_indices[..] strictly
 * ascending in [0, cols); row_offsets[0] == 0, nondecreasing.
 * col_indices may be NULL when every non-empty row is full (its columns are
 * then 0..cols-1 in order, which is the only canonical full row).
 * touched_rows (optional): the ascending ids of all rows with at least one
 * entry, n_touched of them (or *d_n_touched when that is given, <= n_touched).
 * Without it the update scans row_offsets over all rows. */
typedef struct spopt_csr {
    int64_t rows, cols;
    const int32_t* row_offsets;  /* device [rows + 1] */
    const int32_t* col_indices;  /* device [nnz] or NULL (full rows) */
    const float* values;         /* device [nnz] */
    const int64_t* touched_rows; /* device [n_touched], optional */
    int64_t n_touched;
    const int64_t* d_n_touched;  /* device, optional */
} spopt_csr;

#define SPOPT_FORMAT_COO 0
#define SPOPT_FORMAT_CSR 1

typedef struct spopt_grad {
    int32_t format; /* SPOPT_FORMAT_COO or SPOPT_FORMAT_CSR */
    spopt_coo coo;
    spopt_csr csr;
} spopt_grad;

/* ---- optimizer handle --------------------------------------------------- */
typedef struct spopt_optimizer* spopt_t;

/* Create an optimizer over caller-owned device state of shape rows x cols
 * (cols == 1 for a 1-D vector), all contiguous:
 *   params        float [rows*cols]
 *   m_or_momentum float [rows*cols] (Adam m; SGD momentum buffer, may be NULL
 *                 when momentum == 0)
 *   v             float [rows*cols] (Adam only; NULL for SGD)
 *   last_step     int32 [rows*cols] (Adam only; NULL for SGD)
 * The caller initialises m = v = momentum = 0 and last_step = 0 before the
 * first step (the reading that makes the first touch at global step t a gap
 * of t).  config points at spopt_adam_config or spopt_sgd_config (copied).
 * The handle owns the config and the global step counter t, starting at 0.
 * Errors: SPOPT_EINVAL (NULL, bad kind, rows*cols <= 0, hyper-parameter out of
 * range), SPOPT_EDEVICE. */
SPOPT_API int sparse_opt_create(spopt_t* out, int32_t kind, const void* config, int64_t rows, int64_t cols,
                      float* params, float* m_or_momentum, float* v, int32_t* last_step);
SPOPT_API void sparse_opt_destroy(spopt_t h);

/* Global step counter (number of successful step calls so far). */
SPOPT_API int64_t sparse_opt_get_step(spopt_t h);
/* Set t, e.g. to resume from a checkpoint of the state arrays.  0 <= t <
 * 2^31 (last_step is int32).  SPOPT_EINVAL otherwise. */
SPOPT_API int sparse_opt_set_step(spopt_t h, int64_t t);

/* Message of the calling thread's last failure ("" if none). */
SPOPT_API const char* sparse_opt_last_error(void);

/* Timing of the update launch (profiling).  With two hipEvent_t handles set
 * (created by the caller, timing enabled), every later sparse_adam_step,
 * sparse_sgd_step and sparse_step_from_lookups call of the calling thread
 * attaches them to the dispatch of the kernel that updates the table
 * (hipExtLaunchKernel), so `begin` takes that kernel's start time and `end`
 * its end time, with no stream packets of their own.  The events stay the
 * caller's; (NULL, NULL) stops it.  Errors: SPOPT_EINVAL when only one is
 * NULL; a failed launch makes the step return SPOPT_EDEVICE as usual. */
SPOPT_API int sparse_opt_set_step_events(void* begin, void* end);

/* ---- canonicalisation --------------------------------------------------- */

/* ---- host-resident state ------------------------------------------------ */

/* State for tables larger than device memory (the DiskSparseAdam README keeps
 * w, m, v and its step counters out of core and moves only the rows a batch
 * touches).  Here the state lives in pinned host memory mapped into the
 * device's address space; the step kernels then read and write, over the
 * host link, only the touched rows.  Pass the device pointers to
 * sparse_opt_create and read_rows as for device memory; the host pointers
 * are for the caller (initial values, checkpoints), and the state they show
 * is current after the stream has been synchronised.
 * sparse_opt_host_alloc: `bytes` of pinned, mapped host memory, zero-filled;
 * *host_ptr for the host, *device_ptr for kernels.  The caller owns it and
 * frees it with sparse_opt_host_free (after the last use on any stream).
 * Errors: SPOPT_EINVAL (NULL outputs, bytes == 0), SPOPT_ENOMEM.
 * sparse_opt_host_device_pointer: the device address of pinned host memory
 * allocated elsewhere (mapped pinned allocations only); SPOPT_EINVAL when the
 * runtime has no device mapping for host_ptr. */
SPOPT_API int sparse_opt_host_alloc(size_t bytes, void** host_ptr, void** device_ptr);
SPOPT_API void sparse_opt_host_free(void* host_ptr);
SPOPT_API int sparse_opt_host_device_pointer(void* host_ptr, void** device_ptr);

/* Bytes of device workspace coo_from_lookups needs for n lookups of `width`
 * values over keys in [0, key_space).  SPOPT_EINVAL for n < 0, width < 1,
 * key_space < 1, or key and position bits together above 64. */
SPOPT_API int sparse_opt_workspace_size(int64_t n, int64_t width, int64_t key_space, size_t* bytes);

/* Raw lookups -> canonical COO (DiskSparseAdam "Safe Duplicate Aggregation &
 * Sorted I/O"; the canonical CooGradient of the optirs_gpu sparse_optimizer
 * page, section "Sparse gradient representations").
 *   ids        device int64 [n], each in [0, key_space)
 *   vals       device float [n * width], row i belongs to ids[i]
 *   out_keys   device int64 [n]: the U distinct ids, strictly ascending
 *   out_vals   device float [n * width]: row k = sum of the rows of all
 *              lookups of out_keys[k]; summation in float32 in a fixed order
 *              (deterministic run to run), not necessarily lookup order
 *   out_counts device int32 [n]: multiplicity of out_keys[k]
 *   d_nunique  device int64 [1]: U
 * Entries k >= U of the outputs are unspecified.  A key whose values sum to
 * zero is kept (present means touched).
 * width == 1 gives a 1-D CooGradient; width == cols with key_space == rows
 * gives full table rows.
 * Workspace: device, at least sparse_opt_workspace_size(n, width, key_space).
 * Errors: SPOPT_EINVAL, SPOPT_EWORKSPACE, SPOPT_EOVERFLOW (n >= 2^30);
 * with SPOPT_VALIDATE also SPOPT_ERANGE (an id outside [0, key_space)) and
 * SPOPT_ENONFINITE.  In trusted mode an out-of-range id is still detected on
 * the device; the call then sets *d_nunique = 0 (an empty gradient) and
 * writes no other output.  The sort and segment kernels coordinate their
 * blocks through bounded device-side waits; the blocks are numbered in the
 * order they start, so a wait only ever waits on a block that is running,
 * and the bound (about a second) is there to turn a library bug into an
 * answer rather than a hang.  A wait that gives up ends the call the same
 * way: *d_nunique = 0, no other output written (under SPOPT_VALIDATE too:
 * the validation reads the inputs before the sort). */
SPOPT_API int coo_from_lookups(const int64_t* ids, const float* vals, int64_t n, int64_t width,
                     int64_t key_space, int64_t* out_keys, float* out_vals, int32_t* out_counts,
                     int64_t* d_nunique, void* workspace, size_t workspace_bytes, void* stream,
                     uint32_t flags);

/* ---- COO <-> CSR (optirs_gpu sparse_optimizer: CsrGradient::from_coo / to_coo) */

/* Canonical COO -> CSR of shape rows x cols.
 *   in->width == 1:    in->dim must be rows*cols; row = idx / cols,
 *                      col = idx % cols.
 *   in->width == cols: in->dim must be rows; entries are full rows.
 *   row_offsets device int32 [rows + 1] (required)
 *   col_indices device int32 [nnz*width] or NULL (only for width == cols:
 *               full rows, columns implicit)
 *   values      device float [nnz*width] or NULL to skip the copy (the CSR
 *               values then ARE in->values, which has the same layout)
 *   touched_rows device int64 [nnz] or NULL; width == cols only: the touched
 *               row ids (a copy of in->indices); d_n_touched (device int64,
 *               or NULL) receives their count.
 * nnz is read on the device from in->d_nnz when given.
 * Errors: SPOPT_EINVAL, SPOPT_ESHAPE, SPOPT_EOVERFLOW (nnz*width >= 2^31);
 * with SPOPT_VALIDATE also SPOPT_ERANGE and SPOPT_ENOTCANON. */
SPOPT_API int csr_from_coo(const spopt_coo* in, int64_t rows, int64_t cols, int32_t* row_offsets,
                 int32_t* col_indices, float* values, int64_t* touched_rows,
                 int64_t* d_n_touched, void* stream, uint32_t flags);

/* Raw lookups of full table rows -> full-row CSR gradient in one call: the
 * same outputs, bit for bit, as coo_from_lookups(ids, vals, n, cols, rows, ...)
 * followed by csr_from_coo on that COO with its values and row ids used in
 * place (DiskSparseAdam "Safe Duplicate Aggregation & Sorted I/O"; the
 * optirs_gpu sparse_optimizer page's CsrGradient::from_coo).  While it numbers the distinct ids, the segment
 * kernel records how many lie below each block of 8192 rows, so the
 * row_offsets blocks need no search, and the combine of tile-crossing sums
 * shares one launch with them.
 *   ids, vals, out_keys, out_vals, out_counts, d_nunique: as coo_from_lookups
 *              with width = cols and key_space = rows.  out_keys[0, U) are
 *              the CSR's touched rows and out_vals its values (U x cols,
 *              row-major).
 *   row_offsets device int32 [rows + 1] (required)
 *   col_indices device int32 [n * cols] or NULL (full rows: 0..cols-1 each)
 * Workspace: device, at least sparse_opt_workspace_size(n, cols, rows).
 * Errors: as coo_from_lookups, plus SPOPT_EINVAL for a NULL row_offsets and
 * SPOPT_EOVERFLOW for n * cols >= 2^31.  In trusted mode an out-of-range id
 * gives U = 0 and all-zero row_offsets. */
SPOPT_API int csr_from_lookups(const int64_t* ids, const float* vals, int64_t n, int64_t rows,
                               int64_t cols, int64_t* out_keys, float* out_vals,
                               int32_t* out_counts, int64_t* d_nunique, int32_t* row_offsets,
                               int32_t* col_indices, void* workspace, size_t workspace_bytes,
                               void* stream, uint32_t flags);

/* CSR -> COO over the flattened rows*cols view: idx[j] = row*cols + col[j],
 * values copied (already ascending, so canonical).
 *   out_indices device int64 [nnz], out_values device float [nnz] or NULL.
 * Errors: SPOPT_EINVAL; with SPOPT_VALIDATE also SPOPT_ENOTCANON, SPOPT_ERANGE. */
SPOPT_API int csr_to_coo(const spopt_csr* in, int64_t* out_indices, float* out_values, void* stream,
               uint32_t flags);

/* ---- optimizer steps ---------------------------------------------------- */

/* One sparse / lazy Adam step: t += 1, then every touched coordinate i is
 * updated (Lazy or DormancyDecay per the handle's config) and
 * last_step[i] = t.  Nothing else is read or written.  An empty gradient
 * still advances t (t counts step calls).
 * COO gradients: width == 1 with dim == rows*cols, or width == cols with
 * dim == rows.  CSR gradients: rows and cols equal the handle's.
 * Errors: SPOPT_EINVAL (NULL, wrong kind, t would reach 2^31), SPOPT_ESHAPE;
 * with SPOPT_VALIDATE also SPOPT_ERANGE, SPOPT_ENOTCANON, SPOPT_ENONFINITE,
 * and SPOPT_EINVAL when a touched coordinate has last_step >= t.  A rejected
 * step writes nothing and leaves t unchanged.  In trusted mode indices outside
 * the state are skipped, never dereferenced. */
SPOPT_API int sparse_adam_step(spopt_t h, const spopt_grad* g, void* stream, uint32_t flags);

/* One sparse SGD step on the touched coordinates (same gradient forms and
 * error rules as sparse_adam_step).  t advances as well. */
SPOPT_API int sparse_sgd_step(spopt_t h, const spopt_grad* g, void* stream, uint32_t flags);

/* Raw lookups of full table rows -> one optimizer step, in one call: the same
 * outputs and the same table, bit for bit, as csr_from_lookups(ids, vals, n,
 * rows, cols, ...) on the handle's rows x cols followed by sparse_adam_step
 * (Adam handle) or sparse_sgd_step (SGD handle) on the CSR it built, with
 * out_keys as the touched-row list (n_touched = n, d_n_touched = d_nunique).
 * The whole of the optirs_gpu sparse_optimizer page's step from a
 * CooGradient: the canonical gradient ("Canonicalisation"), then the touched
 * coordinates' update.  In trusted mode the step's work shares the CSR
 * call's last launch: the combine of sums that cross segment tiles, the
 * update of every touched row and the row_offsets / col_indices blocks run
 * side by side (a tile-crossing row is updated by the block that completes
 * its sum), when cols % 4 == 0 and row_offsets and col_indices are 16-byte
 * aligned; otherwise, and with SPOPT_VALIDATE, it makes the two calls.
 *   Arguments: as csr_from_lookups, with rows and cols the handle's.
 * Errors: those of csr_from_lookups and of the step call; SPOPT_EINVAL for a
 * NULL handle.  A step the validation rejects leaves the table and t as they
 * were; the canonical outputs are written all the same.  In trusted mode an
 * out-of-range id gives U = 0, as csr_from_lookups: no row is updated and t
 * still advances; so does a device-side wait that gives up (see
 * coo_from_lookups).  A caller that must tell such a step from one with no
 * lookups reads *d_nunique after it. */
SPOPT_API int sparse_step_from_lookups(spopt_t h, const int64_t* ids, const float* vals, int64_t n,
                                       int64_t* out_keys, float* out_vals, int32_t* out_counts,
                                       int64_t* d_nunique, int32_t* row_offsets,
                                       int32_t* col_indices, void* workspace,
                                       size_t workspace_bytes, void* stream, uint32_t flags);

/* The same step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * sparse_step_from_lookups without the workspace arguments, its workspace
 * being a fixed 16 MiB array in the library's device data (one copy per GPU,
 * held until the process ends; about 2 MiB is needed for 65,536 lookups of
 * 128 columns on a 10M-row table, 8.2 MiB for 262,144 lookups on 50M rows).
 * The call allocates nothing (no hipMalloc, no allocating library routine).
 * The caller still passes every input and output.  Every call on a GPU uses
 * that GPU's one array, which keeps the last call's contents (the
 * canonicalisation clears what it accumulates into, so nothing needs
 * clearing beforehand): calls that overlap in time on one GPU, e.g. on two
 * streams without an ordering between them, race and give wrong results.
 * Trusted mode only.
 * Errors: those of sparse_step_from_lookups; SPOPT_EINVAL for SPOPT_VALIDATE
 * or a bad n; SPOPT_EWORKSPACE, before any device work, when the lookups
 * need more scratch than the array holds (sparse_opt_workspace_size(n, cols,
 * rows) > 16 MiB). */
SPOPT_API int sparse_step_from_lookups_noalloc(spopt_t h, const int64_t* ids, const float* vals,
                                               int64_t n, int64_t* out_keys, float* out_vals,
                                               int32_t* out_counts, int64_t* d_nunique,
                                               int32_t* row_offsets, int32_t* col_indices,
                                               void* stream, uint32_t flags);

/* ---- forward gather ----------------------------------------------------- */

/* DiskSparseAdam README, API reference, read_rows(indices): the current rows of
 * a table for a batch of lookups.  out[k*cols + j] = params[indices[k]*cols + j]
 * for k < n, j < cols; duplicates allowed.
 * params: device, rows x cols float32 (e.g. the params of an optimizer handle);
 * indices: device int64[n]; out: device float32[n x cols], caller-owned.
 * Stream-ordered after any step on the same stream, so it reads the updated
 * table.  Trusted mode: an index outside [0, rows) gives a row of zeros and
 * nothing outside the table is read.  SPOPT_VALIDATE: SPOPT_ERANGE for such an
 * index and SPOPT_ENONFINITE for a gathered row holding a NaN or inf (a
 * corrupted row), nothing written.  n == 0 does nothing.
 * Errors: SPOPT_EINVAL (NULL pointers, rows or cols < 1, n < 0). */
SPOPT_API int read_rows(const float* params, int64_t rows, int64_t cols, const int64_t* indices,
                        int64_t n, float* out, void* stream, uint32_t flags);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_OPT_H */
