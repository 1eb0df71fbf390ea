/*
 * libgemmepi -- dense fp16/bf16 GEMM with a fused epilogue for AMD Instinct
 * MI355X (gfx950).
 *
 *   out[M,N] = epilogue( A[M,K] . B  (+ bias) )
 *
 * computed with fp32 accumulation on the MFMA units; the epilogue runs on
 * the accumulator registers and the result is written to HBM once.  This is
 * the computation of the pages' cuBLASLt/nvmath "epilog" mechanism: the bias
 * add (and activation) happens on chip instead of in separate kernels that
 * each re-read the GEMM result from global memory ("nvmath-python cuBLASLt
 * bias fusion guide", sections "Core API and parameter configuration" and
 * "Performance principles and expected gains"; ops-nn MatMul fusion article,
 * section "Level 1: basic fusion").
 *
 * The interface mirrors the pages' stateful Matmul object: planning is a
 * separate, cached step whose cost is amortised over many executions
 * ("nvmath-python cuBLASLt bias fusion guide", section "Advanced techniques
 * and engineering practice", resource reuse; "Fusing bias addition with
 * matrix multiplication using nvmath-python", paragraphs 3 and 5).
 *
 * Conventions (all calls):
 *   - Matrices are row-major.  A is [M,K] (K contiguous).  B is [K,N]
 *     (N contiguous), or [N,K] (K contiguous) with GEMMEPI_FLAG_B_TRANS,
 *     which is the x.W^T orientation of a linear layer with W stored
 *     [out,in].  out is [M,N].
 *   - Device pointers are HIP device pointers on the current device; the
 *     caller owns every buffer.  The library never allocates device memory
 *     at run time; its only device memory is the static scratch of
 *     gemmepi_execute_noalloc, allocated by the code-object loader.
 *   - Every call returns a status and never aborts or prints;
 *     gemmepi_last_error() returns a thread-local description of the last
 *     failure.
 */
#ifndef GEMMEPI_H
#define GEMMEPI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 1.1.0: the stats buffer of gemmepi_execute_norm grew to
 * gemmepi_norm_stats_bytes(M) (32 M bytes and row counters, was 16 M) for the
 * single-pass norm; GEMMEPI_FLAG_NORM_TWO_PASS added. */
#define GEMMEPI_VERSION 110

typedef enum {
  GEMMEPI_OK = 0,
  GEMMEPI_ERR_INVALID_VALUE = 1, /* bad size, enum, flag or null pointer   */
  GEMMEPI_ERR_MISALIGNED = 2,    /* pointer or contiguous dim not aligned  */
  GEMMEPI_ERR_UNSUPPORTED = 3,   /* valid but not implemented combination  */
  GEMMEPI_ERR_DEVICE = 4,        /* pointer not device memory (VALIDATE)   */
  GEMMEPI_ERR_HIP = 5,           /* HIP runtime / launch error             */
  GEMMEPI_ERR_NO_MEMORY = 6      /* host allocation of a plan failed       */
} gemmepi_status_t;

typedef enum {
  GEMMEPI_F16 = 0, /* IEEE binary16 inputs and output */
  GEMMEPI_BF16 = 1 /* bfloat16 inputs and output      */
} gemmepi_dtype_t;

/*
 * The epilogues.  Names follow the MatmulEpilog members the pages name
 * (BIAS, RELU_BIAS, GELU_BIAS: "nvmath-python cuBLASLt bias fusion guide",
 * sections "Core API and parameter configuration" and "Advanced techniques
 * and engineering practice"; RELU_AUX_BIAS: "Fusing bias addition with
 * matrix multiplication using nvmath-python", paragraph 4; DRELU_BGRAD: the
 * same "Advanced techniques" section, backward propagation).
 * acc = A.B in fp32; z = acc + bias; every result is rounded once
 * (round-to-nearest-even) to the output dtype.
 */
typedef enum {
  GEMMEPI_EPI_DEFAULT = 0,       /* out = acc                                  */
  GEMMEPI_EPI_BIAS = 1,          /* out = z                                    */
  GEMMEPI_EPI_RELU_BIAS = 2,     /* out = z > 0 ? z : 0                        */
  GEMMEPI_EPI_RELU_AUX_BIAS = 3, /* RELU_BIAS, plus aux mask bit = (z > 0)    */
  GEMMEPI_EPI_GELU_BIAS = 4,     /* out = 0.5 z (1 + erf(z / sqrt 2))          */
  GEMMEPI_EPI_DRELU_BGRAD = 5,   /* out = mask ? acc : 0; bgrad[n] = sum_m out */
  /* Structural fusion (ops-nn MatMul fusion article, section "Level 2:
   * structural fusion"): y = acc + bias + residual, then a norm over each
   * row of y (all N columns).  Executed with gemmepi_execute_norm only. */
  GEMMEPI_EPI_BIAS_RES_RMSNORM = 6,   /* out = y / sqrt(mean(y^2) + eps) * gamma      */
  GEMMEPI_EPI_BIAS_RES_LAYERNORM = 7, /* out = (y - mean) / sqrt(var + eps) * gamma
                                         + beta; var biased (1/N)                  */
  /* The GELU counterparts of RELU_AUX_BIAS and DRELU_BGRAD (the pages name
   * the ReLU pair for training; these follow the same pattern for GELU). */
  GEMMEPI_EPI_GELU_AUX_BIAS = 8, /* GELU_BIAS, plus z (rounded) kept in aux     */
  GEMMEPI_EPI_DGELU_BGRAD = 9    /* out = acc * gelu'(z_aux); bgrad[n] = sum_m out,
                                    gelu'(z) = Phi(z) + z phi(z)               */
} gemmepi_epilogue_t;

enum {
  /* B is stored [N,K] (K contiguous) instead of [K,N]. */
  GEMMEPI_FLAG_B_TRANS = 1u << 0,
  /* bias is indexed by the column n (length N) instead of the row m
   * (length M, the pages' (m,1) column broadcast over the result's columns). */
  GEMMEPI_FLAG_BIAS_PER_COL = 1u << 1,
  /* Run the unfused baseline instead: the GEMM writes acc to out, then
   * separate elementwise kernels add the bias and apply the activation in
   * place, each reading and writing out in global memory (the three-step
   * sequence of "Fusing bias addition ...", paragraph 1, and of the ops-nn
   * article, section "Level 1: basic fusion"). */
  GEMMEPI_FLAG_UNFUSED = 1u << 2,
  /* execute() checks that every pointer is device memory of the current
   * device (the pages require all operands on one device: "Fusing bias
   * addition ...", paragraph 5). Costs a few host calls. */
  GEMMEPI_FLAG_VALIDATE = 1u << 3,
  /* Never use the thin-M decode kernel; always use the tiled MFMA GEMM. */
  GEMMEPI_FLAG_NO_DECODE = 1u << 4,
  /* Let plan() split K over several workgroups per output tile (split-K)
   * when the shape has too few output tiles to fill the 256 CUs.  Such a
   * plan needs a device workspace (gemmepi_workspace_bytes) and runs
   * through gemmepi_execute_ws.  No effect on the decode kernel and the
   * norm epilogues. */
  GEMMEPI_FLAG_SPLIT_K = 1u << 5,
  /* Let plan() stage B stored [K,N] (no B_TRANS): each execution first
   * copies B into a K-contiguous [N,K] copy in the workspace, then runs the
   * GEMM on it.  The copy reads and writes N K elements once; plan() takes
   * it only for GEMMs of at least 8192 rows that do not split K, where the
   * GEMM on K-contiguous B (slabs read with 128-bit LDS reads rather than
   * transposing ones) gains more than the copy costs.  Such a plan needs a
   * device workspace (gemmepi_workspace_bytes) and runs through
   * gemmepi_execute_ws.  No effect with B_TRANS, on the decode kernel and on
   * the norm epilogues. */
  GEMMEPI_FLAG_STAGE_B = 1u << 6,
  /* gemmepi_execute_norm: always run the two-kernel form (the GEMM writes y,
   * rounded to the dtype, then a second kernel normalises it in place)
   * instead of the single pass.  For comparison and testing. */
  GEMMEPI_FLAG_NORM_TWO_PASS = 1u << 7
};

/* Opaque, reference-counted handle to a cached plan. */
typedef struct gemmepi_plan_s* gemmepi_plan_t;

/*
 * Plan one GEMM shape.  Pure host work, no HIP call: validates the
 * arguments, picks the kernel (tiled MFMA GEMM, or the thin-M decode kernel
 * for M <= 16 with B_TRANS, never for the norm epilogues) and its tile
 * configuration from the shape, and
 * returns a handle from a process-wide cache keyed on all arguments
 * (planning the same key again returns the same handle with its reference
 * count raised).
 *
 *   plan   out: the handle (set to NULL on failure)
 *   M,N,K  1 .. 2^31-1; K must be a multiple of 8; N must be a multiple of 8
 *          unless GEMMEPI_FLAG_B_TRANS is set (16-byte rows for 128-bit loads)
 *   dtype  GEMMEPI_F16 or GEMMEPI_BF16
 *   epi    one of gemmepi_epilogue_t
 *   flags  OR of GEMMEPI_FLAG_*
 *
 * Errors: INVALID_VALUE (null plan, sizes, unknown enum/flag bits),
 * MISALIGNED (K or N not a multiple of 8 as above), UNSUPPORTED for
 * shapes past the kernels' 32-bit buffer offsets (K >= 2^22, or N >= 2^23
 * with B stored [K,N]: 256 K-contiguous rows, or the 128 k rows of the
 * deepest slab of B, must span less than 2 GiB) or with M * N > 2^40,
 * NO_MEMORY.
 */
gemmepi_status_t gemmepi_plan(gemmepi_plan_t* plan, int64_t M, int64_t N, int64_t K,
                              gemmepi_dtype_t dtype, gemmepi_epilogue_t epi, uint32_t flags);

/*
 * As gemmepi_plan, with an explicit tile configuration of the tiled GEMM
 * (0 <= tile_id < gemmepi_num_tiles(); -1 = heuristic choice, identical to
 * gemmepi_plan).  Used by tuning sweeps and by tests that cover every tile
 * shape.  An explicit tile_id also disables the decode kernel.  The pages'
 * planner picks one of several algorithm candidates for a shape; this call
 * fixes the candidate instead ("nvmath-python cuBLASLt bias fusion guide",
 * section "Advanced techniques and engineering practice").
 * Errors: as gemmepi_plan, plus INVALID_VALUE for an unknown tile_id.
 */
gemmepi_status_t gemmepi_plan_tiled(gemmepi_plan_t* plan, int64_t M, int64_t N, int64_t K,
                                    gemmepi_dtype_t dtype, gemmepi_epilogue_t epi,
                                    uint32_t flags, int32_t tile_id);

/*
 * As gemmepi_plan_tiled, with an explicit K split (split-K): the k slabs of
 * each output tile are divided into `splits` contiguous ranges, each run by
 * its own workgroup; every range writes an fp32 partial tile to the
 * workspace, and the last range of a tile to finish sums the partials in
 * range order (so out does not depend on which finishes last) and applies
 * the epilogue once.  This is the wave-quantisation remedy for shapes with
 * few output tiles and a long K; the pages do not define it.  Its
 * caller-owned workspace follows the workspace argument the pages pass to
 * the vendor library's matmul ("Bias fusion with cuBLASLt in PyTorch
 * inference: fewer kernel launches and memory accesses", body).
 *
 *   splits  1 = no split; 2 .. 64 = that many ranges (fewer when K has
 *           fewer k slabs of the tile); 0 = chosen by plan() with the tile
 *           (as GEMMEPI_FLAG_SPLIT_K)
 *   tile_id -1 = chosen; an explicit tile or splits > 1 disables the
 *           decode kernel
 * Errors: as gemmepi_plan_tiled, plus INVALID_VALUE for splits outside
 * [0, 64], UNSUPPORTED for splits > 1 with a norm epilogue.
 */
gemmepi_status_t gemmepi_plan_split(gemmepi_plan_t* plan, int64_t M, int64_t N, int64_t K,
                                    gemmepi_dtype_t dtype, gemmepi_epilogue_t epi,
                                    uint32_t flags, int32_t tile_id, int32_t splits);

/*
 * Device workspace a plan needs, in bytes (the caller-owned workspace of
 * the vendor library's matmul in "Bias fusion with cuBLASLt in PyTorch
 * inference: fewer kernel launches and memory accesses", body): 0 unless
 * the plan stages B or splits K.  A staged plan needs 2 N K bytes (padded to 256) for the copy of
 * B; a split plan 4 bytes per output tile (arrival counters, padded to 256
 * bytes) plus one fp32 partial tile per (tile, split).  NULL plan: 0.
 */
size_t gemmepi_workspace_bytes(gemmepi_plan_t plan);

/*
 * Enqueue one execution on `stream` (a hipStream_t; NULL = the null
 * stream) and return without synchronising.  No allocation, no host sync.
 *
 *   A     [M,K] dtype, device, 16-byte aligned
 *   B     [K,N] or [N,K] (B_TRANS) dtype, device, 16-byte aligned
 *   bias  BIAS / RELU_BIAS / RELU_AUX_BIAS / GELU_BIAS / GELU_AUX_BIAS:
 *         input, dtype, [M] (or [N] with BIAS_PER_COL), 2-byte aligned;
 *         required.
 *         DRELU_BGRAD / DGELU_BGRAD: OUTPUT, fp32 [N], 4-byte aligned,
 *         overwritten with the column sums of out's unrounded values;
 *         required.
 *         DEFAULT: ignored (may be NULL).
 *   aux   RELU_AUX_BIAS: OUTPUT mask; DRELU_BGRAD: INPUT mask.  uint32
 *         words, [M, gemmepi_aux_ld_words(N)] row-major, 16-byte aligned;
 *         column n of row m is bit (n & 31) of word (m, n >> 5); padding
 *         bits are written as 0 and ignored on input.
 *         GELU_AUX_BIAS: OUTPUT, DGELU_BGRAD: INPUT: the pre-activation z
 *         in the dtype, [M,N] row-major, 16-byte aligned.
 *         Other epilogues: ignored.
 *   out   [M,N] dtype, device, 16-byte aligned; overwritten (in the UNFUSED
 *         path it is also read back by the elementwise kernels).
 *
 * The fused path launches one kernel (DRELU_BGRAD: a tiny bgrad zero-fill
 * kernel, then the GEMM).  bgrad is accumulated with fp32 atomics, so its
 * last bits may differ from run to run; out and aux are bitwise
 * reproducible.
 * Errors: INVALID_VALUE (null plan or required pointer), MISALIGNED,
 * DEVICE (VALIDATE only), HIP (launch failure, e.g. no gfx950 device).
 */
gemmepi_status_t gemmepi_execute(gemmepi_plan_t plan, const void* A, const void* B, void* bias,
                                 void* aux, void* out, void* stream);
/* (A plan with a norm epilogue is rejected by gemmepi_execute with
 * INVALID_VALUE; it runs through gemmepi_execute_norm below.  A plan that
 * splits K or stages B is rejected too: it runs through gemmepi_execute_ws.) */

/*
 * gemmepi_execute with a caller-owned device workspace, which a plan that
 * splits K or stages B needs (gemmepi_workspace_bytes > 0); the vendor library's matmul
 * likewise takes its workspace from the caller ("Bias fusion with cuBLASLt
 * in PyTorch inference", body).  For a plan that does not split K it is
 * identical to gemmepi_execute and the workspace is ignored.  A staged plan
 * overwrites the workspace's copy of B on every execution.
 *
 *   workspace        device memory, 256-byte aligned, at least
 *                    gemmepi_workspace_bytes(plan) bytes.  Its counter
 *                    area must be zero before its first use: zero the whole
 *                    workspace once after allocating it.  Every execution
 *                    leaves the counters at zero again, so a workspace can
 *                    be reused by later executions of any plan on the same
 *                    stream; executions that may overlap (other streams)
 *                    need workspaces of their own.
 *   workspace_bytes  its size
 * The partial tiles are summed in split order, so out and aux stay bitwise
 * reproducible.
 * Errors: as gemmepi_execute, plus INVALID_VALUE (workspace missing or too
 * small), MISALIGNED (workspace), DEVICE (VALIDATE: workspace not device
 * memory of the current device).
 */
gemmepi_status_t gemmepi_execute_ws(gemmepi_plan_t plan, const void* A, const void* B, void* bias,
                                    void* aux, void* out, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): as
 * gemmepi_execute_ws, but a plan that splits K takes its workspace from a
 * static device array of the library, gemmepi_noalloc_scratch_bytes()
 * bytes (80 MiB) per device, which the code-object loader allocates when
 * the library's kernels are first loaded on a device and which stays
 * allocated until the process ends.  The call itself allocates nothing.
 * Its arrival counters are cleared by a fill kernel at the start of each
 * call (the array keeps the previous call's contents).  For a plan that
 * does not split K it is identical to gemmepi_execute.
 *
 * Every call on one device shares that device's array: calls that may
 * overlap on one device (other streams, other threads) race on it and
 * give wrong results; serialise them, or give each its own workspace
 * through gemmepi_execute_ws.
 *
 * Arguments as gemmepi_execute.  Errors: as gemmepi_execute, plus
 * UNSUPPORTED when the plan's workspace (gemmepi_workspace_bytes: split-K
 * partials, or a staged copy of B) exceeds the static array, HIP when its
 * device address cannot be looked up.
 */
gemmepi_status_t gemmepi_execute_noalloc(gemmepi_plan_t plan, const void* A, const void* B,
                                         void* bias, void* aux, void* out, void* stream);

/* Size in bytes of the per-device static scratch of gemmepi_execute_noalloc. */
size_t gemmepi_noalloc_scratch_bytes(void);

/*
 * Measured tile choice for a tiled-GEMM plan: the pages' planner "tries
 * multiple algorithms" and keeps the best ("nvmath-python cuBLASLt bias
 * fusion guide", section "Advanced techniques and engineering practice";
 * "Fusing bias addition ...", paragraph 5).  Executes the plan with every
 * tile configuration on the caller's operands (one warm-up and `reps` timed
 * runs each, HIP events on `stream`), then waits for the stream.  The plan
 * is switched to the fastest tile in place (plan_info then says "tuned"),
 * later gemmepi_plan calls for the same M, N, K, dtype, epilogue and flags
 * use it, and with GEMMEPI_TUNE_CACHE=<file> the choice is written to that
 * text file, which the first gemmepi_plan of a later process reads.
 *
 *   A..out   as gemmepi_execute; out, aux and bgrad are overwritten
 *   reps     1 .. 10000
 *   times_ms NULL, or gemmepi_num_tiles() floats receiving each tile's mean
 *            milliseconds per execution
 * Not thread-safe against executions of the same plan on other threads.
 * Errors: INVALID_VALUE (null plan, reps, a plan made with an explicit
 * tile), UNSUPPORTED (decode, norm, split-K or B-staging plans), the errors of
 * gemmepi_execute, HIP (timing, or the cache file could not be written).
 */
gemmepi_status_t gemmepi_autotune(gemmepi_plan_t plan, const void* A, const void* B, void* bias,
                                  void* aux, void* out, int32_t reps, float* times_ms,
                                  void* stream);

/*
 * Enqueue one execution of a plan made with GEMMEPI_EPI_BIAS_RES_RMSNORM or
 * GEMMEPI_EPI_BIAS_RES_LAYERNORM (ops-nn MatMul fusion article, section
 * "Level 2: structural fusion": MatMul + bias + residual + norm as one
 * operator; the residual joins before the norm, eps sits inside the square
 * root, the variance is the biased one):
 *
 *   y[m,:]   = A[m,:] . B + bias[:] + residual[m,:]
 *   out[m,:] = (y[m,:] - mean_m) * rstd_m * gamma[:] (+ beta[:])
 *   LAYERNORM: mean_m = mean(y[m,:]), rstd_m = 1 / sqrt(var(y[m,:]) + eps)
 *   RMSNORM:   mean_m = 0,            rstd_m = 1 / sqrt(mean(y[m,:]^2) + eps)
 *
 * Single pass (the default, when the plan's whole grid of workgroups fits
 * on the device at once): y stays in the GEMM kernel's fp32 registers and is
 * never rounded before the norm; the workgroups that share a band of rows
 * add fp64 partial row sums of y and y^2 into the stats workspace, wait
 * until the whole band has arrived, then each normalises its own tile and
 * writes out once.  Otherwise (a larger grid, or GEMMEPI_FLAG_NORM_TWO_PASS)
 * two kernels: the GEMM writes y (rounded once to the dtype) into out and
 * adds the row sums, then a second kernel normalises each row of out in
 * place.  With GEMMEPI_FLAG_UNFUSED the GEMM writes A.B, and separate
 * kernels add the bias, add the residual and normalise (statistics from
 * the row itself).
 *
 *   A, B      as gemmepi_execute (B [K,N], or [N,K] with B_TRANS)
 *   bias      dtype [N] (always per column), 2-byte aligned, or NULL (none)
 *   residual  dtype [M,N] row-major, 16-byte aligned, or NULL (none)
 *   gamma     dtype [N], 2-byte aligned; required
 *   beta      dtype [N], 2-byte aligned, or NULL (none); ignored by RMSNORM
 *   eps       > 0, finite
 *   stats     gemmepi_norm_stats_bytes(M) bytes, 8-byte aligned; the
 *             caller's workspace during the call.  On return its first
 *             16 M bytes are fp64 [M][2]: row m holds (mean_m, rstd_m).
 *             A fused execution clears the rest; the 32-bit word at byte
 *             offset 32 M then reads 1 after a single pass and 0 after two
 *             kernels (UNFUSED leaves it as it was); if its bit 1 is
 *             set, a workgroup of the single pass stopped waiting for its
 *             band of rows (bounded at a few seconds; it cannot happen when
 *             the grid is resident as required) and wrote NaN rows.  The
 *             environment variable GEMMEPI_NORM_WAIT_POLLS (0 to 2^21 polls,
 *             read at every call) lowers that bound, to test this path.
 *             Calls that share one stats buffer must not overlap.
 *   out       dtype [M,N], 16-byte aligned; overwritten (in the two-kernel
 *             form it holds y between the two kernels)
 * Errors: INVALID_VALUE (null plan or required pointer, not a norm plan,
 * eps not positive and finite), MISALIGNED, DEVICE (VALIDATE), HIP.
 */
gemmepi_status_t gemmepi_execute_norm(gemmepi_plan_t plan, const void* A, const void* B,
                                      const void* bias, const void* residual,
                                      const void* gamma, const void* beta, float eps,
                                      void* stats, void* out, void* stream);

/* Bytes of the stats buffer of gemmepi_execute_norm for M rows: 32 M for
 * (mean, rstd) and the row sums, plus one 32-bit word per 64 rows and a
 * status word, rounded up to 16; 0 for M < 1.  The statistics of the MatMul + Norm operator of the ops-nn
 * MatMul fusion article, section "Level 2: structural fusion". */
size_t gemmepi_norm_stats_bytes(int64_t M);

/* Drop one reference; the plan is freed when the last reference goes: the
 * release of the Matmul object's resources ("Fusing bias addition with
 * matrix multiplication using nvmath-python", paragraph 5).
 * Errors: INVALID_VALUE for NULL or a handle that is not live. */
gemmepi_status_t gemmepi_plan_destroy(gemmepi_plan_t plan);

/* Human-readable description of the plan (path, tile, grid) into buf
 * (NUL-terminated, truncated to len): which candidate the planner chose
 * ("nvmath-python cuBLASLt bias fusion guide", section "Advanced techniques
 * and engineering practice").  Errors: INVALID_VALUE. */
gemmepi_status_t gemmepi_plan_info(gemmepi_plan_t plan, char* buf, size_t len);

/* Number of tile configurations of the tiled GEMM, and the name
 * ("BMxBNxBK_wWMxWN_sNS_pSCHED_mMFMA") of one of them (NULL for an unknown
 * id): the algorithm candidates the planner chooses among ("nvmath-python
 * cuBLASLt bias fusion guide", section "Advanced techniques and engineering
 * practice"). */
int32_t gemmepi_num_tiles(void);
const char* gemmepi_tile_name(int32_t tile_id);

/* Mask row pitch in uint32 words for N columns: ceil(N/32) rounded up to a
 * multiple of 4 (16 bytes); and the mask size in bytes for M rows.
 * Return 0 for N < 1 (or M < 1).  The mask is the ReLU auxiliary output of
 * "Fusing bias addition with matrix multiplication using nvmath-python",
 * paragraph 4, which gives no layout; this bit-packed one is the library's. */
int64_t gemmepi_aux_ld_words(int64_t N);
size_t gemmepi_aux_bytes(int64_t M, int64_t N);

/* Static string for a status code ("unknown status" for others): the
 * library's form of the runtime error the pages raise for invalid operands
 * ("Fusing bias addition with matrix multiplication using nvmath-python",
 * paragraph 5). */
const char* gemmepi_status_string(gemmepi_status_t s);

/* Thread-local description of the most recent failure in this thread
 * ("" if none).  Valid until the next failing call in the same thread. */
const char* gemmepi_last_error(void);

/* GEMMEPI_VERSION of the built library (library bookkeeping; no passage of
 * the pages defines it). */
int32_t gemmepi_version(void);


#ifdef __cplusplus
}
#endif

#endif /* GEMMEPI_H */
