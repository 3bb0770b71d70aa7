/*
 * gemm.h: C ABI of the MI355X (gfx950) tiled GEMM with a fused register epilogue.
 *
 *   D = act(alpha * op(A) * op(B) + beta * C + bias[j])
 *
 * The operation is the GEMM C = alpha*A*B + beta*C of "CUTLASS: Fast Linear Algebra in CUDA
 * C++" (section "Efficient Matrix Multiplication on GPUs"), with the element-wise post-processing
 * of that page's section "Fusing Element-wise Operations: An Example with SGEMM" (scale by alpha,
 * add a bias term and beta times the C element, clamp with max(0, .)) and the bias vector of
 * "Flexible Performant GEMM Kernels on GPUs", section 5.3, added to every row of the product.
 * Mixed precision follows that paper's section 2.3: 16-bit inputs with 32-bit accumulation
 * (fp16/bf16 -> fp32; int8 -> int32 here).  The API has two steps, as that paper's section 6
 * describes for cuBLASLt: build a plan for one problem description, then launch it any number of
 * times with different buffers and scalars.
 *
 * Storage: every matrix is ROW-MAJOR.  op = GEMM_OP_N uses the stored array as is; GEMM_OP_T
 * means the stored array is the transpose of the operand.
 *   op_a = N: A is M x K, element (i,k) at A[i*lda + k], lda >= K.
 *   op_a = T: A is stored K x M, op(A)(i,k) = A[k*lda + i], lda >= M.
 *   op_b = N: B is K x N, element (k,j) at B[k*ldb + j], ldb >= N.
 *   op_b = T: B is stored N x K, op(B)(k,j) = B[j*ldb + k], ldb >= K.
 *   C and D are M x N with the same leading dimension ldc >= N.
 * Leading dimensions are counted in elements of each matrix's own type.  No alignment is
 * required; 16-byte aligned pointers and leading dimensions take the faster load paths.
 *
 * Supported type combinations (ab_type -> cd_type); bias is fp32 for float inputs and int32
 * for int8 inputs; C has the type of D; accumulation is fp32 (int32 for int8):
 *   F32 -> F32,  F16 -> F16 | F32,  BF16 -> BF16 | F32,  I8 -> I32,
 *   CF16 -> CF32 | CF16,  DF16 -> DF32 | DF16  (epilogue NONE only; alpha and beta are real
 *   and scale both parts; no transforms or diagonal operands).
 * Conversion to a 16-bit output rounds to nearest even.
 *
 * Ownership: the caller owns every device buffer and keeps it alive until the stream work that
 * uses it has finished.  A plan is a small host object, destroyed with gemm_plan_destroy.  Most
 * plans hold no device memory and may be shared between host threads and streams.  A plan that
 * splits K over workgroups ("ksplit S" in its description: a short product, M <= 64, or a
 * product with few output tiles and a long K) owns a split-K workspace (S * M * N floats per
 * product of the batch) on the device of its first gemm_run, allocated by that call and freed
 * by gemm_plan_destroy: its runs must not overlap in time (use one plan per concurrent stream).
 * The first run of a skinny split-K plan ("gemm_skinny... ksplit S") must not be captured into a
 * graph (later runs may be); the first run of a fast-kernel split-K plan inside a capture runs
 * unsplit.  A split run enqueues the partial products and a finishing kernel.
 * A 16- or 8-bit plan on the fast kernel (large and mid-size products) whose operand rows are
 * off the 16-byte grid (an odd leading
 * dimension or batch stride, an unaligned pointer at run time, or an M/N-contiguous row length
 * that is not a multiple of 16 bytes), or with a load transform on op(A) or op(B), first copies
 * those operands into aligned, zero-padded rows of a workspace it owns (about the size of the
 * copied operands; the copy applies the transform), then runs the direct-load kernel on the
 * copies: two kernels per run ("repack A/B/AB" in the description when the plan itself calls
 * for the copy).  With A stored transposed and B not, A's copy is made transposed, into
 * K-contiguous rows ("(A to K-major)"), and it is also made for an A that could be read in
 * place when the product is wide enough to repay it (see GEMM_ALGO_FAST_KMAJOR).  The
 * workspace is allocated by the first run that needs it on a device (not
 * while the stream is captured: such a run reads the operands in place with a slower kernel,
 * same results) and freed by gemm_plan_destroy; runs of one such plan must not overlap in time.
 * Likewise a complex or dual plan large enough for the real fast kernel ("as real 2x2 blocks"
 * in its description) owns a workspace for op(B) rewritten as real 2 x 2 blocks (twice B's
 * bytes) and, when A is transposed, A split into parts; its runs enqueue the rewrite and then
 * the real product, and a run without that workspace uses the complex kernel.  A graph that
 * captured runs of a plan holding a workspace reads and writes that workspace when replayed:
 * destroy such a plan only after the graphs that captured it.
 *
 * Errors: every function returns a status; nothing throws across this boundary.  gemm_run is
 * asynchronous: it validates, enqueues its kernels on `stream` and returns (one kernel; or,
 * as above, a copy or rewrite pass, the product, and a finishing kernel when K is split: up to
 * three); faults during execution surface at the caller's next synchronisation.
 */
#ifndef TGE_GEMM_H
#define TGE_GEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GEMM_OP_N = 0, GEMM_OP_T = 1 } gemm_op_t;

/*
 * Element types.  The complex and dual types are pairs stored interleaved (first part, then
 * second part of each number, 2 x 16 or 2 x 32 bits): complex x = re + im*i with i^2 = -1, dual
 * x = re + eps*d with eps^2 = 0 ("Flexible Performant GEMM Kernels on GPUs", section 5.4).  A
 * leading dimension or stride of such a matrix counts numbers, not parts.
 */
typedef enum {
    GEMM_F32 = 0,
    GEMM_F16 = 1,
    GEMM_BF16 = 2,
    GEMM_I8 = 3,
    GEMM_I32 = 4,
    GEMM_CF16 = 5,   /* complex, fp16 parts */
    GEMM_CF32 = 6,   /* complex, fp32 parts */
    GEMM_DF16 = 7,   /* dual, fp16 parts */
    GEMM_DF32 = 8    /* dual, fp32 parts */
} gemm_dtype_t;

/* bias: bias[j] added to every row; relu: max(0, .) applied last. */
typedef enum {
    GEMM_EPI_NONE = 0,
    GEMM_EPI_RELU = 1,
    GEMM_EPI_BIAS = 2,
    GEMM_EPI_BIAS_RELU = 3
} gemm_epilogue_t;

typedef enum {
    GEMM_STATUS_SUCCESS = 0,
    GEMM_STATUS_INVALID_VALUE = 1, /* a bad argument: negative size, ld too small, NULL pointer */
    GEMM_STATUS_NOT_SUPPORTED = 2, /* a valid request this library does not implement */
    GEMM_STATUS_HIP_ERROR = 3,     /* the HIP runtime reported an error at launch */
    GEMM_STATUS_ALLOC_FAILED = 4,  /* memory could not be allocated: host memory for a plan
                                      (plan creation), or device memory for a plan's split-K
                                      workspace (gemm_run) */
    GEMM_STATUS_SCRATCH_LIMIT = 5  /* gemm_run_noalloc: the run needs more scratch than
                                      GEMM_NOALLOC_SCRATCH_BYTES */
} gemm_status_t;

/* Bytes of device scratch each device holds for gemm_run_noalloc (64 MiB). */
#define GEMM_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * Element-wise transforms applied to operand values as they are loaded, before they enter the
 * product or the epilogue: the "transform" component of "Flexible Performant GEMM Kernels on
 * GPUs" (section 4), which applies a function to every element after a load, e.g. an
 * activation, and the "bias + ReLU on C & D" variant of that paper's section 5.3 (Table 2).
 *   GEMM_TRANSFORM_RELU replaces every element whose sign bit is set by +0, i.e. max(x, 0) for
 *   every non-NaN x (-0 becomes +0; a NaN keeps its value unless its sign bit is set).
 * The type conversions of that section ("a type conversion after a load"), for op(A) and op(B)
 * of a 16-bit plan (ab_type F16 or BF16) with dense operands:
 *   GEMM_TRANSFORM_FROM_F32  the operand is stored as fp32 (its leading dimension and batch
 *                            stride count fp32 elements) and every element is rounded to the
 *                            nearest ab_type value, ties to even, as it is loaded;
 *   GEMM_TRANSFORM_FROM_I8   the operand is stored as int8 and converted exactly.
 * A plan with a conversion converts those operands, once per run, into 16-bit rows of a
 * workspace it owns ("convert A/B from f32/i8" in its description), allocated by its first run
 * on a device (that run must not be captured into a graph: it returns NOT_SUPPORTED there) and
 * freed by gemm_plan_destroy; its runs must not overlap in time.  Then the product runs on the
 * converted rows as the same plan without the conversion would.
 */
typedef enum {
    GEMM_TRANSFORM_NONE = 0,
    GEMM_TRANSFORM_RELU = 1,
    GEMM_TRANSFORM_FROM_F32 = 2,
    GEMM_TRANSFORM_FROM_I8 = 3
} gemm_transform_t;

/*
 * Kind of an operand.  GEMM_OPERAND_DIAGONAL: the operand is a square diagonal matrix given by
 * the vector of its diagonal elements (ab_type; a diagonal A is M x M with K == M, a diagonal B
 * is N x N with K == N); its op and leading dimension are ignored.  Off-diagonal elements are
 * never loaded and K steps that meet no diagonal element are skipped: the diagonal layout and
 * the skip predicate of "Flexible Performant GEMM Kernels on GPUs", section 5.2 (Table 1).
 */
typedef enum { GEMM_OPERAND_DENSE = 0, GEMM_OPERAND_DIAGONAL = 1 } gemm_operand_t;

/*
 * Kernel choice of a plan.  GEMM_ALGO_AUTO lets the plan choose from the shape, types and
 * layouts (the rule is described by gemm_plan_describe's text); the others pin a route, for
 * comparisons and tests, and fall back to the general kernel where the pinned route's
 * preconditions do not hold:
 *   FAST         the fast kernel (16- and 8-bit inputs; 256x256 tiles, 128x128 with a tile of
 *                128), with its K split when the plan's rule asks for one;
 *   FAST_STAGED  the fast kernel, reading operands that are off the 16-byte grid in place
 *                through registers instead of copying them first;
 *   GENERAL      the general tiled kernel, never the fast, skinny or split routes;
 *   SKINNY       the memory-bound kernel for M <= 64 wherever its preconditions hold (op(A) = A,
 *                16-byte aligned rows, K a whole number of 64-byte chunks; 16-bit inputs, or
 *                int8 with B transposed);
 *   SPLIT        the fast kernel with K split into any number >= 2 of whole-slab chunks;
 *   NOSPLIT      the plan's own choice without a K split;
 *   FAST_KMAJOR  as FAST, and with A stored transposed and B not, A is first copied transposed
 *                into K-contiguous rows so that the kernel of the non-transposed layout runs
 *                (GEMM_ALGO_AUTO makes that copy when the product is wide enough to repay it,
 *                and always when A has to be copied anyway).
 */
typedef enum {
    GEMM_ALGO_AUTO = 0,
    GEMM_ALGO_FAST = 1,
    GEMM_ALGO_FAST_STAGED = 2,
    GEMM_ALGO_GENERAL = 3,
    GEMM_ALGO_SKINNY = 4,
    GEMM_ALGO_SPLIT = 5,
    GEMM_ALGO_NOSPLIT = 6,
    GEMM_ALGO_FAST_KMAJOR = 7
} gemm_algo_t;

typedef struct gemm_plan *gemm_plan_t;

/*
 * Full problem description for gemm_plan_create_desc.  The first twelve fields are the
 * arguments of gemm_plan_create; batch and the strides are those of gemm_plan_create_batched
 * (batch 1 and zero strides for a single product); transform_a / transform_b act on op(A) and
 * op(B) (zero-padding past the edges is unaffected), transform_c on C before it is scaled by
 * beta (NONE or RELU: C has the type of D); kind_a / kind_b make an operand diagonal (see gemm_operand_t; a diagonal operand's
 * stride_a / stride_b moves its vector); algo pins the kernel route (see gemm_algo_t;
 * GEMM_ALGO_AUTO for the plan's own choice) and tile the workgroup tile of the general kernel
 * (256, 128 or 64; 0 for the plan's own choice; 256 also selects the fast kernel where it
 * applies, and 128 with GEMM_ALGO_AUTO or FAST its 128 x 128 tiles for 16-bit and int8 inputs,
 * read in place or from the aligned copies; the plan's own choice takes those for mid-size
 * products); batch2 and the stride2 fields add a second batch mode (0 or 1: none): the launch
 * computes batch x batch2 products, product (b1, b2) reading and writing every operand moved by
 * b1 * stride + b2 * stride2 elements (a zero stride broadcasts the operand along that mode),
 * the index map of a tensor contraction whose batch index has two modes with their own
 * strides ("Flexible Performant GEMM Kernels on GPUs", section 4: layouts that reorganise
 * indices as they load).  The D's of all products must be disjoint: the mode with the smaller
 * C/D stride has a stride of at least one D ((M-1)*ldc + N), the other at least that stride
 * times the smaller mode's count.  Two-mode plans read their operands in place (no aligned
 * copies, conversions or complex rewrites: a conversion returns NOT_SUPPORTED).  Plain data:
 * the library keeps no pointer to it.
 */
typedef struct {
    int64_t M, N, K;
    gemm_op_t op_a, op_b;
    int64_t lda, ldb, ldc;
    gemm_dtype_t ab_type, cd_type;
    gemm_epilogue_t epilogue;
    int64_t batch;
    int64_t stride_a, stride_b, stride_c, stride_bias;
    gemm_transform_t transform_a, transform_b, transform_c;
    gemm_operand_t kind_a, kind_b;
    gemm_algo_t algo;
    int32_t tile;
    int64_t batch2;
    int64_t stride2_a, stride2_b, stride2_c, stride2_bias;
} gemm_desc_t;

/*
 * Builds a plan for one problem description.  Host-only: makes no HIP call.
 *   out            receives the plan; set to NULL on any failure.
 *   M, N, K        problem size, each >= 0.  M == 0 or N == 0 is a valid empty problem;
 *                  K == 0 gives D = act(beta*C + bias).
 *   op_a, op_b     GEMM_OP_N or GEMM_OP_T (see the storage rules above).
 *   lda, ldb, ldc  leading dimensions in elements, at least the stored row length (and >= 1).
 *   ab_type        type of A and B;  cd_type: type of C and D (see the supported table).
 *   epi            epilogue kind.
 * Returns INVALID_VALUE for negative sizes, leading dimensions below the minimum, an enum out of
 * range or out == NULL; NOT_SUPPORTED for a type pair outside the table or when a matrix spans
 * 2^31 bytes or more.  The kernel and workgroup tile are chosen from the shape (see
 * gemm_plan_create_desc to pin them).
 */
gemm_status_t gemm_plan_create(gemm_plan_t *out, int64_t M, int64_t N, int64_t K, gemm_op_t op_a,
                               gemm_op_t op_b, int64_t lda, int64_t ldb, int64_t ldc,
                               gemm_dtype_t ab_type, gemm_dtype_t cd_type, gemm_epilogue_t epi);

/*
 * Strided-batched plan: `batch` independent products of the same shape in one launch,
 *   D_b = act(alpha*op(A_b)*op(B_b) + beta*C_b + bias_b),  b = 0 .. batch-1,
 * where X_b starts stride_x elements (of X's own type) after X_{b-1}: A_b = A + b*stride_a,
 * B_b = B + b*stride_b, C_b = C + b*stride_c and D_b = D + b*stride_c (C and D share the
 * stride, as they share ldc), bias_b = bias + b*stride_bias.  This is the simplest of the
 * logical-index-to-offset mappings that "Flexible Performant GEMM Kernels on GPUs" (section 4)
 * builds with its layout component for batched and tensor-contraction operands.
 *   batch          number of products, >= 0 (0 is a valid empty launch).
 *   stride_a, stride_b, stride_bias   >= 0; 0 shares the operand between all products.
 *   stride_c       0 when batch <= 1, else at least the span of one D ((M-1)*ldc + N), so
 *                  that products never write the same element.
 * The other arguments and the errors are those of gemm_plan_create, plus INVALID_VALUE for a
 * negative batch or stride or an overlapping stride_c, and NOT_SUPPORTED when the launch would
 * need 2^31 workgroups or more.  gemm_run then takes the pointers of product 0.
 */
gemm_status_t gemm_plan_create_batched(gemm_plan_t *out, int64_t M, int64_t N, int64_t K,
                                       gemm_op_t op_a, gemm_op_t op_b, int64_t lda, int64_t ldb,
                                       int64_t ldc, gemm_dtype_t ab_type, gemm_dtype_t cd_type,
                                       gemm_epilogue_t epi, int64_t batch, int64_t stride_a,
                                       int64_t stride_b, int64_t stride_c, int64_t stride_bias);

/*
 * Builds a plan from a full description (see gemm_desc_t): every option of gemm_plan_create
 * and gemm_plan_create_batched plus the load transforms,
 *   D_b = act(alpha * tA(op(A_b)) * tB(op(B_b)) + beta * tC(C_b) + bias_b).
 * Returns the errors of gemm_plan_create_batched, plus INVALID_VALUE for desc == NULL, a
 * transform, operand kind or algorithm out of range (a conversion on C included), a tile other
 * than 0, 256, 128 or 64, or a diagonal operand that is not square (K != M for A, K != N for B);
 * NOT_SUPPORTED for a conversion on a plan whose ab_type is not F16 or BF16, or on a diagonal
 * or complex operand.  The span limit applies to a converted operand in its stored type.
 */
gemm_status_t gemm_plan_create_desc(gemm_plan_t *out, const gemm_desc_t *desc);

/*
 * Enqueues D = act(alpha*op(A)*op(B) + beta*C + bias) on `stream` (a hipStream_t; NULL is the
 * null stream of the current device).  All pointers are device pointers on the current device.
 *   A, B     operands (may be NULL only if the product is empty: M, N or K == 0).
 *   C        read only when beta != 0 (may be NULL, or hold NaN, when beta == 0).  C == D is
 *            allowed (in-place update); any other overlap between D and an input is undefined.
 *   D        output, required when M > 0 and N > 0.
 *   bias     N elements (fp32, or int32 for int8 inputs); required when the plan's epilogue
 *            includes a bias, ignored otherwise.
 * For a batched plan every pointer is that of product 0 (see gemm_plan_create_batched).
 *   alpha, beta  scalars applied in fp32 (int8 plans require alpha == 1 and beta in {0, 1}).
 * Returns INVALID_VALUE for a NULL plan, a missing required pointer or a NaN scalar,
 * NOT_SUPPORTED for int8 scalars outside the rule above or for the first run of a skinny split-K
 * plan or of a converting plan (GEMM_TRANSFORM_FROM_*) during stream capture, ALLOC_FAILED when
 * that first run cannot allocate its workspace
 * (the plans that copy or rewrite operands, or split K for the fast kernel, run without their
 * workspace instead), HIP_ERROR when a launch fails.  M == 0, N == 0 or a batch of 0 returns
 * SUCCESS without launching.
 */
gemm_status_t gemm_run(gemm_plan_t plan, const void *A, const void *B, const void *C, void *D,
                       const void *bias, float alpha, float beta, void *stream);

/*
 * gemm_run for callers that cannot allocate device memory: code being captured into a HIP
 * graph, tight serving loops, harnesses that forbid allocation.  Same arguments, results and
 * errors as gemm_run, and the same kernels, but no call allocates or frees memory (no hipMalloc,
 * no plan-owned workspace is created or used): the split-K partial sums, the aligned operand
 * copies and the complex/dual operand rewrites that gemm_run keeps in plan-owned workspaces are
 * placed in a scratch array of GEMM_NOALLOC_SCRATCH_BYTES that the library holds on every
 * device it runs on (from the first call there until the process ends).  A run whose route
 * needs more than that returns GEMM_STATUS_SCRATCH_LIMIT before anything is enqueued.  Nothing
 * in the scratch needs to start at zero: every run writes the regions it reads.  A copy that a
 * plan makes only by choice (the transposed copy of an A it could read in place) is skipped,
 * reading A in place, when it does not fit beside the run's other regions.  All calls on a
 * device share its one array, so calls whose device work overlaps in time (other streams, or
 * host threads) race on it and give undefined results: serialise them on one stream.  The
 * plan itself is only read.  The first call on a device that needs scratch looks up the array's
 * address there (a HIP runtime query, which may load the library's device code on that device):
 * make that first call outside a stream capture; later calls may be captured.  HIP_ERROR also
 * covers a failure of that lookup.
 */
gemm_status_t gemm_run_noalloc(gemm_plan_t plan, const void *A, const void *B, const void *C,
                               void *D, const void *bias, float alpha, float beta, void *stream);

/* Frees a plan and its workspace, if any (waiting for the device work that may use it).  NULL is
 * a no-op.  Always returns SUCCESS. */
gemm_status_t gemm_plan_destroy(gemm_plan_t plan);

/* Static, human-readable name of a status code (never NULL). */
const char *gemm_status_string(gemm_status_t status);

/*
 * Describes the kernel a plan launches: writes a NUL-terminated text such as
 * "mfma f16->f16 NN tile 256x256x64 waves 2x2 grid 1024" into buf (at most len bytes).
 * Returns INVALID_VALUE for a NULL plan or buffer.
 */
gemm_status_t gemm_plan_describe(gemm_plan_t plan, char *buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* TGE_GEMM_H */
