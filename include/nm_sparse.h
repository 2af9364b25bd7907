/*
 * nm_sparse.h -- C ABI of libnmsparse.so: batch-one N:M semi-structured sparse
 * matrix-vector product y = W x on AMD Instinct MI355X (gfx950).
 *
 * Sources (the pages, cited by title and section):
 *   [NEWS-NEW] news.bitwarelabs.com, "SparseDecoding: decoding-aware pruning for
 *              accurate and fast LLM generation", section "What's new": decoding at
 *              batch one is memory-bandwidth bound and dominated by sparse
 *              matrix-vector products; N:M semi-structured sparsity keeps N weights
 *              of every M consecutive ones; the SpMV uses bitmask indexing and
 *              fixed-step traversal.
 *   [KERNEL]   aimodeling.com SparseDecoding article, section "The Kernel Is the
 *              Other Half of the Answer": a 32-bit mask word per 32 input columns,
 *              exactly 16 set bits per word at 50% sparsity, replacing per-nonzero
 *              32-bit column indices; 2:4, 4:8, 8:16 and 16:32 all keep half the
 *              weights and move the same metadata; speedups are quoted against the
 *              dense product.
 *
 * Format (the packed layout every entry point shares):
 *   W        fp16 [rows][cols] row-major (out x in, y = W x), cols % 32 == 0.
 *   masks    uint32 [rows][cols/32]; bit j (LSB = 0) of word w of row r is set iff
 *            W[r][32w + j] is kept. Every word has exactly V = 32*N/M set bits (16 for
 *            the 50% patterns, 8 for the 25% ones) and every aligned group of M columns
 *            exactly N.
 *   values   fp16 [rows][cols*N/M]; the kept weights of row r, word by word, in
 *            ascending column order, so word w's values start at V*w of the row.
 *   Patterns: 2:4, 4:8, 8:16, 16:32 (50%, the ones the pages measure) and 1:4, 2:8,
 *            4:16, 8:32 (25%; [NEWS-NEW] states the method for N:M in general).
 *   x        fp16 [cols];  y  fp16 [rows].
 *   fp16 is passed as its raw bit pattern (uint16_t).
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller. The library never
 *     allocates, frees, copies to the host or synchronises.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default stream).
 *     Work is enqueued on it and the call returns at once.
 *   - Arguments are validated before any HIP call; an invalid call returns a status
 *     code and enqueues nothing. Calls never abort, print or throw.
 *   - A fault inside a kernel is not reported by the call; it surfaces at the
 *     caller's next synchronisation on the stream.
 *   - Outputs must not alias inputs (documented, not checked).
 *   - Thread-safe and reentrant; the only state is a per-device cache of device
 *     attributes.
 */
#ifndef NM_SPARSE_H
#define NM_SPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NM_OK = 0,
  NM_ERR_NULL = 1,     /* a required pointer is NULL                                   */
  NM_ERR_SHAPE = 2,    /* rows < 1, cols < 32, cols % 32 != 0, batch / tokens < 1, or a
                          size beyond an entry point's limits                         */
  NM_ERR_PATTERN = 3,  /* (N, M) not a supported pattern (nm_spmm: 50% patterns for
                          batch > 1; nm_spmm_prefill: 2:4, 4:8, 8:16)                 */
  NM_ERR_ALIGN = 4,    /* W, values or x not 16-byte aligned; masks not 4-byte; y not 2 */
  NM_ERR_TOO_WIDE = 5, /* 2*cols bytes of x exceed the LDS one workgroup may use        */
  NM_ERR_HIP = 6,      /* a HIP runtime call failed (see nm_last_hip_error)             */
  NM_ERR_SCRATCH = 7   /* nm_spmm_noalloc: the shape's column split needs more than the
                          library's static scratch (NM_NOALLOC_SCRATCH_BYTES)              */
} nm_status;

/* Number of fp16 values of the packed matrix: rows*cols*N/M; 0 if the arguments are
 * invalid. Pure host function. */
size_t nm_values_count(int64_t rows, int64_t cols, int N, int M);

/* Number of uint32 mask words: rows*cols/32; 0 if the arguments are invalid. */
size_t nm_masks_count(int64_t rows, int64_t cols);

/* Widest x (in columns, a multiple of 32) that nm_spmv and nm_gemv_dense accept on
 * the current HIP device, from its per-workgroup LDS size; 0 if no device. */
int64_t nm_max_cols(void);

/* Encoder ([NEWS-NEW] N-of-M selection, [KERNEL] bitmask format).
 * In each aligned group of M columns keep the N weights of largest magnitude, where
 * the magnitude of an fp16 weight is its bit pattern with the sign bit cleared,
 * compared as an unsigned integer (so -0 == +0, and +-Inf ranks below every NaN);
 * equal magnitudes go to the lower column. Writes `masks` and `values` as described
 * above, copying the kept bits exactly. W: [rows][cols] fp16 bits; values:
 * nm_values_count() elements; masks: nm_masks_count() words. Bit-exact and
 * deterministic. */
int nm_pack(const uint16_t* W, uint16_t* values, uint32_t* masks,
            int64_t rows, int64_t cols, int N, int M, void* stream);

/* Decoder, the inverse of nm_pack ([KERNEL] bitmask format): writes the dense matrix W'
 * [rows][cols] fp16 that (values, masks) describe: the kept values at their columns (the
 * value of set bit j of word w is the one after the set bits below j), +0 elsewhere.
 * Bit-exact and deterministic. A mask word with the wrong number of set bits gives an
 * unspecified W' but no access outside the inputs. For prompt-sized products of 4:8, 8:16
 * and 16:32, whose sparse prefill kernels are slower than the dense one (they keep half the
 * bytes, not half the instructions), decoding once and using nm_gemm_dense_prefill is the
 * fastest route where a dense copy fits. values, W 16-byte aligned; masks 4-byte. */
int nm_unpack(const uint16_t* values, const uint32_t* masks, uint16_t* W,
              int64_t rows, int64_t cols, int N, int M, void* stream);

/* Sparse product ([NEWS-NEW], [KERNEL]): y[r] = fp16( sum_c W'[r][c] * x[c] ), where W'
 * is the matrix the packed (values, masks) describe. Products and sums are fp32; y is
 * rounded once to fp16 (round to nearest even). The summation order is fixed, so the
 * result is bit-identical from run to run. Masks must be as nm_pack writes them; a
 * malformed mask gives an unspecified y but never an out-of-bounds access. */
int nm_spmv(const uint16_t* values, const uint32_t* masks, const uint16_t* x, uint16_t* y,
            int64_t rows, int64_t cols, int N, int M, void* stream);

/* Several sparse products that share one input x, in one launch ([NEWS-NEW]: every
 * linear layer of a decoding step is a batch-one sparse product; q, k and v, or gate and
 * up, read the same activation): y[k][r] = fp16( sum_c W'_k[r][c] * x[c] ) for
 * k < count, 1 <= count <= NM_MAX_SPMV_GROUP, each as nm_spmv computes it. values, masks, y
 * and rows are HOST arrays of `count` entries: product k's packed matrix (device pointers),
 * its output (device pointer, rows[k] elements) and its row count; all share cols, N:M and
 * x (device, cols elements). The arrays are read during the call only. One launch covers
 * every product when cols <= 8192 and the pattern is 2:4, 4:8, 8:16 or 16:32, with the
 * workgroup shape nm_spmv would give their rows together; then each y is bit-identical to
 * nm_spmv's when nm_spmv alone runs the same number of waves per row and not its
 * narrow-layer path (every product of 4096 columns, for instance), and within the same
 * tolerance of the exact product otherwise. Other shapes and patterns take one nm_spmv
 * launch per product.
 * Alignment as nm_spmv; the outputs must not alias each other or the inputs. Status codes
 * as nm_spmv, with NM_ERR_SHAPE also for count outside 1..NM_MAX_SPMV_GROUP. Allocates
 * nothing. */
#define NM_MAX_SPMV_GROUP 8
int nm_spmv_group(int count, const uint16_t* const* values, const uint32_t* const* masks,
                  const uint16_t* x, uint16_t* const* y, const int64_t* rows, int64_t cols,
                  int N, int M, void* stream);

/* Dense baseline, the denominator of the pages' speedups ([KERNEL]):
 * y[r] = fp16( sum_c W[r][c] * x[c] ) with fp32 products and sums, fixed order. */
int nm_gemv_dense(const uint16_t* W, const uint16_t* x, uint16_t* y,
                  int64_t rows, int64_t cols, void* stream);

/* Batch sparse product (the matrix-matrix side of the SpMV / SpMM split that [NEWS-NEW]
 * draws: prefill and larger batches run matrix-matrix products), for the same packed
 * matrix and batch >= 1 activation vectors:
 *   Y[b][r] = fp16( sum_c W'[r][c] * X[b][c] ),  X fp16 [batch][cols], Y fp16 [batch][rows]
 * (row b of X is one activation vector: the layout of a batch of tokens). Products and
 * sums fp32, one RNE rounding, fixed summation order (bit-identical run to run).
 *   - batch >= 32 with 2:4, 4:8 or 8:16: nm_spmm_prefill (matrix cores), with its limits,
 *     except 32..48 vectors on layers of at most 4096 rows and 32 on layers of at most
 *     8192 rows where nm_spmm_skinny takes the layer (next item): there 16-vector
 *     launches measured faster than the prefill kernel.
 *   - 5 <= batch < 32 where it was measured faster than the small-batch kernel (2:4 on
 *     layers of at least 256 rows; 4:8 and 8:16 on layers of at least 2048 rows, and on
 *     smaller ones from 9 or 12 vectors): nm_spmm_skinny, 16 vectors per launch, each
 *     launch routed by the same rule at its own count (17..20 vectors: the last 1..4 on
 *     the small-batch kernel).
 *   - 16:32 from 64 vectors: nm_spmm_prefill (fragments expanded for the dense matrix
 *     instruction), with its limits.
 *   - 16:32 from 5 to 63 vectors, per launch of up to 16 vectors: nm_spmm_skinny's
 *     expansion kernel for a launch of at least 14 vectors on layers of at least 2048 rows
 *     (4096 if wider than 4096 columns), or of at least 12 on layers of at least 4096 rows
 *     and at most 4096 columns; the small-batch kernel for the other launches (e.g. 24
 *     vectors: one launch of 16 expanded, 8 on the small-batch one).
 *   - otherwise the small-batch kernel (vector units; x staged in LDS in column phases
 *     when it does not fit at once, so any width is accepted), on consecutive groups of
 *     8 rows of X (one launch per group). batch == 1 gives the same result as nm_spmv
 *     within the tolerance of the product (it may use another summation order).
 * The 25% patterns are accepted for batch == 1 only (and cols <= nm_max_cols()); larger
 * batches of them return NM_ERR_PATTERN. X must be 16-byte aligned, Y 2-byte aligned;
 * batch < 1 or above 2^24 is NM_ERR_SHAPE. */
int nm_spmm(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y,
            int64_t rows, int64_t cols, int64_t batch, int N, int M, void* stream);

/* nm_spmm with a caller-owned workspace. The same Y definition as nm_spmm. Where
 * nm_spmm_workspace_bytes(...) for the same arguments is > 0 and workspace_bytes is at least
 * that, work that would leave most CUs idle is split over more workgroups:
 *   - skinny launches (50% patterns at 5..16 vectors per launch, nm_spmm's route) on layers
 *     too short to fill the GPU (e.g. 1024 rows): the columns of each 16-row tile go to 2, 4
 *     or 8 workgroups;
 *   - batches of more than 16 vectors (any 50% pattern) whose output tiles of 64 rows x 32
 *     (up to 32 vectors) or 64 vectors are too few to fill the GPU (mid-size batches: e.g.
 *     up to 256 tokens on 4096 x 4096): instead of nm_spmm's route, one launch of the
 *     prefill kernel with each tile's columns split over 2 .. 8 workgroups, whole blocks of
 *     512 columns each ([NEWS-NEW]: batched tokens run matrix-matrix products); the same
 *     for 16:32 batches of 12 .. 16 vectors on layers of at most 2048 rows;
 *   - prompts of more than 128 tokens (any 50% pattern) where a model of the kernels' step
 *     times puts it well ahead: tiles of 128 x 128 or 256 x 128 (2:4 only) with their
 *     columns split over 2 .. 8 workgroups, at most one workgroup per CU (e.g. 4096 x 14336
 *     at 256 .. 1024 tokens).
 * In both the last-arriving workgroup of a tile sums the fp32 partial tiles in split order
 * (fixed, so bit-identical run to run, but not bit-identical to nm_spmm's order: the same
 * tolerance against the exact product). workspace: device memory, 16-byte aligned, owned by
 * the caller; its first 4 * CU-count bytes, rounded up to 256 (1 KiB on MI355X), are
 * counters that must be zero before the first call on it (e.g. one hipMemset when
 * allocated); every call leaves them zero again, so one workspace serves any sequence of
 * shapes on the device. NULL or a smaller workspace runs nm_spmm's kernels (no error; a
 * prompt whose taller split does not fit takes the 64-row split where that applies and
 * fits). Calls
 * that use one workspace must be ordered (one stream): overlapping calls on it race. Other
 * arguments and errors as nm_spmm; a misaligned workspace is NM_ERR_ALIGN. */
int nm_spmm_ws(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y,
               int64_t rows, int64_t cols, int64_t batch, int N, int M, void* workspace,
               size_t workspace_bytes, void* stream);

/* Bytes of workspace nm_spmm_ws can use for these arguments on the current device; 0 when
 * the shape takes no split (or the arguments are invalid, or no device): the counters, then
 * the partial tiles, 1 KiB per 16-row tile and split on the skinny kernels (at most 257 KiB
 * on MI355X), 8 or 16 KiB per 64-row tile and split on the prefill kernel (the grid within
 * two workgroups per CU: at most 8 MiB + 1 KiB on MI355X), 64 or 128 KiB per 128- or 256-row
 * tile and split on the taller splits (one workgroup per CU: at most 32 MiB + 1 KiB). */
size_t nm_spmm_workspace_bytes(int64_t rows, int64_t cols, int64_t batch, int N, int M);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): nm_spmm_ws with its workspace in a
 * static device array of the library, NM_NOALLOC_SCRATCH_BYTES per GPU, held from the first
 * call on that GPU until the process ends. The same arguments, routing, Y and errors as
 * nm_spmm_ws with a workspace of that size; a shape whose split needs more
 * (nm_spmm_workspace_bytes > NM_NOALLOC_SCRATCH_BYTES; none on MI355X, whose largest is
 * 32 MiB + 1 KiB) is NM_ERR_SCRATCH before any launch. Calls no hipMalloc/hipFree. The first call
 * on a GPU looks the array up (hipGetSymbolAddress) and queues a fill kernel that clears it
 * on `stream`, ahead of its own kernels; the kernels leave the counters at zero after every
 * call. All calls on one GPU share the array: calls that overlap on one GPU (other streams,
 * other threads, without ordering between them) race and give unspecified Y. */
#define NM_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u + 4096u)
int nm_spmm_noalloc(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y,
                    int64_t rows, int64_t cols, int64_t batch, int N, int M, void* stream);

/* The batch product of nm_spmm on the matrix instructions for any batch >= 1, whatever
 * nm_spmm's routing would pick (the same Y definition, summation in the instructions' fixed
 * order, bit-identical run to run), for the 50% patterns: 2:4 on the 2:4 sparse instruction
 * directly; 4:8 and 8:16 as two 2:4 operands per 4-column group (its first two kept values,
 * and the rest); 16:32, whose 16 kept values may sit anywhere in a 32-column word, with each
 * word's values expanded to dense 32-column fragments for the dense instruction. X is
 * staged in LDS in column phases, 16 vectors per launch. Limits: cols <= 2^21, batch <= 2^24
 * (NM_ERR_SHAPE beyond); other patterns are NM_ERR_PATTERN. Masks must be as nm_pack writes
 * them; a malformed mask gives an unspecified Y but never an out-of-bounds access. values
 * and X 16-byte aligned, masks 4-byte, Y 2-byte. Allocates nothing. */
int nm_spmm_skinny(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y,
                   int64_t rows, int64_t cols, int64_t batch, int N, int M, void* stream);

/* Dense counterpart of nm_spmm, the same-GPU baseline of the batch product:
 * Y[b][r] = fp16( sum_c W[r][c] * X[b][c] ) with fp32 products and sums, fixed order.
 * batch >= 32: nm_gemm_dense_prefill; below: the small-batch kernel, 8 vectors per launch. */
int nm_gemm_dense(const uint16_t* W, const uint16_t* X, uint16_t* Y,
                  int64_t rows, int64_t cols, int64_t batch, void* stream);

/* Prefill product of a packed 50% matrix on the sparse matrix cores ([NEWS-NEW]: prefill
 * is compute-bound and runs sparse matrix-matrix products; [KERNEL]: that is where 2:4
 * sparse matrix hardware speeds inference up, and the bitmask format): for tokens >= 1
 * rows of X,
 *   Y[t][r] = fp16( sum_c W'[r][c] * X[t][c] ),  X fp16 [tokens][cols], Y fp16 [tokens][rows],
 * with the (values, masks) of nm_pack for a 50% pattern, (N, M) = (2, 4), (4, 8), (8, 16) or
 * (16, 32) (others are NM_ERR_PATTERN). 2:4 runs on the 2:4 sparse instruction directly; 4:8
 * and 8:16, which keep 8 values in every 16 columns, as two 2:4 operands per 4-column group
 * (its first two kept values, and the rest), so at twice the instruction count; 16:32, whose
 * 16 kept values may sit anywhere in a word's 32 columns, on the dense instruction with each
 * lane's 8 columns expanded from its mask byte ([KERNEL]: the bitmask gives every kept
 * value's column). fp16 products, fp32 sums
 * in the matrix instruction's order (fixed, so bit-identical run to run), one RNE
 * rounding. Limits: cols <= 2^21, tokens <= 2^24 (NM_ERR_SHAPE beyond). Masks must be as
 * nm_pack writes them; a malformed mask gives an unspecified Y but never an out-of-bounds
 * access. values, X 16-byte aligned; masks 4-byte; Y 2-byte. */
int nm_spmm_prefill(const uint16_t* values, const uint32_t* masks, const uint16_t* X, uint16_t* Y,
                    int64_t rows, int64_t cols, int64_t tokens, int N, int M, void* stream);

/* Dense counterpart of nm_spmm_prefill on the dense matrix cores, the same-GPU baseline of
 * the prefill product: Y[t][r] = fp16( sum_c W[r][c] * X[t][c] ), fp32 sums in the
 * instruction's fixed order. Same limits and alignment as nm_spmm_prefill (W 16-byte). */
int nm_gemm_dense_prefill(const uint16_t* W, const uint16_t* X, uint16_t* Y,
                          int64_t rows, int64_t cols, int64_t tokens, void* stream);

/* Introspection: the name of the kernel nm_spmm launches for this shape, batch and pattern
 * on the current device (for more than one launch, the kernel of the first); "" if the
 * arguments are invalid. Static string, never NULL. */
const char* nm_spmm_variant(int64_t rows, int64_t cols, int64_t batch, int N, int M);

/* Introspection: the name of the kernel nm_spmm_ws launches for these arguments with a
 * workspace of nm_spmm_workspace_bytes (the column-split kernels where it takes them, else as
 * nm_spmm_variant); "" if the arguments are invalid. Static string, never NULL. */
const char* nm_spmm_ws_variant(int64_t rows, int64_t cols, int64_t batch, int N, int M);

/* Introspection: the name of the kernel configuration nm_spmm_prefill (sparse == 1: 2:4;
 * sparse == 2: 4:8 or 8:16; sparse == 3: 16:32) or nm_gemm_dense_prefill (sparse == 0)
 * launches for this shape
 * on the current device, as it appears in profiler traces (for example
 * "prefill_spmm_kernel<4, 8, 64, 2>"); "" if the arguments are invalid. Static string,
 * never NULL. */
const char* nm_prefill_variant(int64_t rows, int64_t cols, int64_t tokens, int sparse);

/* Introspection: the name of the kernel configuration nm_spmv launches for this shape
 * and pattern on the current device, as it appears in profiler traces (for example
 * "spmv_kernel<2, 4, true, 1>"); "" if the arguments are invalid. Static
 * string, never NULL. Used by the benchmark to attribute measured durations. */
const char* nm_spmv_variant(int64_t rows, int64_t cols, int N, int M);

/* Introspection: the workgroup shape nm_spmv uses for this shape on the current device.
 * Writes shape[0] = rows per workgroup, shape[1] = groups of 8 rows per workgroup,
 * shape[2] = waves per row group (each takes a contiguous range of the columns),
 * shape[3] = number of workgroups (ceil(rows / shape[0])). Validates like nm_spmv. */
int nm_spmv_launch_shape(int64_t rows, int64_t cols, int N, int M, int64_t* shape);

/* Static description of a status code; never NULL. */
const char* nm_status_string(int status);

/* The raw hipError_t behind the last NM_ERR_HIP returned on the calling thread. */
int nm_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NM_SPARSE_H */
