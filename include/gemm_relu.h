/*
 * gemm_relu.h -- C ABI of the MI355X (gfx950) fp16 GEMM with a fused ReLU
 * (and the same GEMM with a fused bias + GELU epilogue).
 *
 * Operation (the GEMM + ReLU example of "Writing high-performance kernels in
 * TileLang", section "Escribamos un GEMM"): for fp16 matrices A (M x K) and
 * B (K x N),
 *
 *     C[i][j] = fp16( max( sum_k A[i][k] * B[k][j], 0 ) )
 *
 * The products are accumulated in fp32 (the example's accumulator type), the
 * ReLU is applied to the fp32 accumulator, and the result is rounded once to
 * fp16, to nearest with ties to even (a sum past the fp16 range becomes +inf).
 * The order of the fp32 additions is unspecified. An empty sum (K = 0) gives
 * C = 0. Inputs are expected to be finite.
 *
 * Layout: A, B and C are dense row-major device buffers of IEEE binary16
 * values with leading dimensions K, N and N. No torch or HIP types appear in
 * this header; a stream is passed as an opaque pointer (a hipStream_t, or
 * NULL for the null stream).
 *
 * Ownership: the caller owns A, B and C and keeps them alive until the work
 * enqueued on `stream` has finished. The library neither frees nor retains
 * them. C must not overlap A or B.
 *
 * Execution: the call validates its arguments on the host, enqueues one kernel
 * on `stream` and returns without waiting. Faults during execution surface at
 * the caller's next synchronisation of that stream. Calls on different streams
 * may run concurrently.
 *
 * Workspace: for few rows (M <= 64) the K dimension is split across
 * workgroups, whose fp32 partial sums meet in a library-owned workspace
 * (partials plus one counter per output tile; K is not split when one
 * split's M x N fp32 partials would reach 2 GiB). The library allocates it with
 * hipMalloc on the first such call for a (device, stream) pair, clears its
 * counters with an asynchronous memset on that stream, keeps it until the
 * process ends, and grows it (to at least twice its size) when a later call
 * needs more. A replaced workspace is kept, not freed, until the process
 * ends, because a HIP graph captured on that stream earlier may still use
 * it. Each launch leaves the counters at zero, so calls on one
 * stream reuse it in order; calls on different streams use different
 * workspaces. Two host threads enqueueing on the same stream at the same
 * time race on the workspace. Failure to allocate gives GEMM_RELU_ENOMEM.
 * Creating or growing a workspace is refused with GEMM_RELU_EUNSUPPORTED
 * while the stream is being captured into a HIP graph (it allocates and
 * clears memory); make one call of the same or a larger shape on that stream
 * before capturing. Calls that fit the existing workspace capture normally.
 *
 * Errors: every entry point returns a gemm_relu_status. All argument checks
 * happen before any HIP runtime call, so a rejected call has no side effects.
 */
#ifndef GEMM_RELU_H
#define GEMM_RELU_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gemm_relu_status {
    GEMM_RELU_OK = 0,
    /* a dimension is negative, a pointer is NULL while its matrix is not
       empty, or C overlaps A or B */
    GEMM_RELU_EINVAL = 1,
    /* a dimension exceeds INT32_MAX, a pointer is not 2-byte aligned, the
       current device is not gfx950, or opts names an unknown tile */
    GEMM_RELU_EUNSUPPORTED = 2,
    /* the HIP runtime reported an error (no device, launch failure) */
    GEMM_RELU_EHIP = 3,
    /* a library-owned workspace could not be allocated */
    GEMM_RELU_ENOMEM = 4,
    /* gemm_relu_f16_noalloc only: the launch needs more scratch than the
       library's fixed array holds (see GEMM_RELU_NOALLOC_MAX_*) */
    GEMM_RELU_ETOOBIG = 5
} gemm_relu_status;

/* Pass as gemm_relu_opts.tile to let the library choose. */
#define GEMM_RELU_TILE_AUTO (-1)

/*
 * Block orders for gemm_relu_opts.block_order. GEMM_RELU_ORDER_DEFAULT with
 * group_m > 0 is always the XCD-aware grouped order; with group_m = 0 the
 * library picks the order (gemm_relu_default_order says which).
 */
#define GEMM_RELU_ORDER_DEFAULT 0   /* XCD-aware grouped order, or the library's pick */
#define GEMM_RELU_ORDER_ROW_MAJOR 1 /* plain row-major tile order */

/*
 * Optional launch choices. They change speed, never the set of admissible
 * results. Zero-initialise and set only what you need; tile = -1 means auto.
 */
typedef struct gemm_relu_opts {
    int32_t tile;        /* GEMM_RELU_TILE_AUTO or an id < gemm_relu_tile_count() */
    int32_t block_order; /* GEMM_RELU_ORDER_* */
    int32_t group_m;     /* tile-rows per group of the grouped order; 0 = default */
    int32_t reserved[5]; /* must be zero */
} gemm_relu_opts;

/*
 * C = ReLU(A @ B) in fp16, as described at the top of this header.
 *   M, N, K : matrix sizes, each in [0, INT32_MAX]
 *   A       : device pointer to M*K fp16 values (row-major, leading dim K)
 *   B       : device pointer to K*N fp16 values (row-major, leading dim N)
 *   C       : device pointer to M*N fp16 values (row-major, leading dim N),
 *             fully overwritten
 *   stream  : hipStream_t to enqueue on, or NULL
 * M == 0 or N == 0 is a successful no-op (no launch).
 */
int gemm_relu_f16(int64_t M, int64_t N, int64_t K,
                  const void* A, const void* B, void* C, void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * operation, arguments, layout, ownership and errors as gemm_relu_f16, and
 * the same kernels and results, but the call allocates nothing (no hipMalloc,
 * no hipFree, no memset): where gemm_relu_f16 would use its per-stream
 * split-K workspace, this entry point uses a fixed array that the library
 * holds on each GPU until the process ends, of
 *     GEMM_RELU_NOALLOC_MAX_TILES x 4 bytes of counters plus
 *     GEMM_RELU_NOALLOC_MAX_PARTIAL_BYTES of fp32 partial sums.
 * A launch that splits K across workgroups (few rows, or few output tiles
 * of the split-K tiles of 16, 32 or 64 rows x 128 columns) over more output
 * tiles than GEMM_RELU_NOALLOC_MAX_TILES, or with more partial sums than
 * GEMM_RELU_NOALLOC_MAX_PARTIAL_BYTES (splits x M x N x 4 bytes), is refused
 * with GEMM_RELU_ETOOBIG before any HIP call; other shapes need no scratch
 * and have no such limit. Every call on one GPU shares
 * that GPU's array: calls that may run at the same time on one GPU (on
 * different streams, or from several host threads) race on it and must be
 * ordered by the caller. The first call on a GPU enqueues one extra small
 * kernel that clears the counters; each launch leaves them at zero.
 */
#define GEMM_RELU_NOALLOC_MAX_TILES 4096
#define GEMM_RELU_NOALLOC_MAX_PARTIAL_BYTES (2 * 1024 * 1024)
int gemm_relu_f16_noalloc(int64_t M, int64_t N, int64_t K,
                          const void* A, const void* B, void* C, void* stream);

/* Same as gemm_relu_f16; opts (may be NULL) pins the tile and block order. */
int gemm_relu_f16_ex(int64_t M, int64_t N, int64_t K,
                     const void* A, const void* B, void* C, void* stream,
                     const gemm_relu_opts* opts);

/*
 * C = GELU(A @ B + bias) in fp16: the fused epilogue of "TileLang simplifica
 * la creación de kernels GPU de alto rendimiento" (section "Fusionar
 * operaciones para reducir viajes a memoria"), where the bias addition and
 * the GELU run on the accumulator in registers and C is written once:
 *
 *     C[i][j] = fp16( GELU( sum_k A[i][k] * B[k][j] + bias[j] ) )
 *
 * with GELU(x) = x * Phi(x), Phi the standard normal distribution function
 * (the definition; no tanh approximation). The products are accumulated in
 * fp32, the bias is added in fp32, GELU is evaluated in fp32 and the result
 * rounded once to fp16, to nearest even.
 *   bias : device pointer to N fp16 values, one per column of C (read only;
 *          may be NULL only if N == 0; must not overlap C)
 * All other arguments, the layout, ownership, execution and errors are those
 * of gemm_relu_f16 / gemm_relu_f16_ex, with these additions: a NULL bias
 * with N > 0 or a bias overlapping C gives GEMM_RELU_EINVAL, an odd bias
 * address GEMM_RELU_EUNSUPPORTED.
 */
int gemm_bias_gelu_f16(int64_t M, int64_t N, int64_t K,
                       const void* A, const void* B, const void* bias, void* C, void* stream);

/* Same as gemm_bias_gelu_f16; opts (may be NULL) pins the tile and block order. */
int gemm_bias_gelu_f16_ex(int64_t M, int64_t N, int64_t K,
                          const void* A, const void* B, const void* bias, void* C, void* stream,
                          const gemm_relu_opts* opts);

/* A static, human-readable message for a status code. */
const char* gemm_relu_strerror(int status);

/* Number of compiled tile configurations, and the name of one ("" if out of range). */
int gemm_relu_tile_count(void);
const char* gemm_relu_tile_name(int tile);

/* Kernel families of gemm_relu_tile_desc.family. */
#define GEMM_RELU_FAMILY_PIPELINED 0 /* direct-to-LDS loads into a ring of LDS stages */
#define GEMM_RELU_FAMILY_STAGED 1    /* loads through registers into a double-buffered LDS tile */
#define GEMM_RELU_FAMILY_SPLITK 2    /* waves and workgroups split K; fp32 partials are summed */
#define GEMM_RELU_FAMILY_SMALL 3     /* direct-to-LDS loads of whole rows into a ring, small tiles
                                        (operands as stored; transposed ones run the staged kernel) */

/*
 * The launch parameters of one compiled tile: the search space of an offline
 * tuner, which explores tile sizes, the K depth of a step, the pipeline depth
 * and the thread count, and leaves out configurations over the LDS budget
 * ("Writing high-performance kernels in TileLang", sections "GEMM con Tensor
 * Cores y decisiones que cambian la velocidad" and "El ajuste automático
 * encuentra configuraciones específicas para cada GPU"). Every compiled tile
 * already fits the 160 KiB of LDS of a gfx950 compute unit; configurations
 * that do not are rejected when the library is compiled.
 */
typedef struct gemm_relu_tile_desc {
    int32_t bm, bn;          /* rows and columns of C per workgroup */
    int32_t bk;              /* K depth of one pipeline step */
    int32_t stages;          /* K steps held per workgroup: LDS ring slots (pipelined), LDS buffers
                                (staged) or register ring depth per wave (split-K) */
    int32_t waves_m, waves_n, waves_k; /* wave grid; waves_k > 1 when the waves split K */
    int32_t threads;         /* threads per workgroup (64 per wave) */
    int32_t lds_bytes;       /* static LDS per workgroup */
    int32_t split_k;         /* 1 when K is also split across workgroups through the workspace */
    int32_t default_group_m; /* tile-rows per group of the grouped order when opts leave it 0 */
    int32_t family;          /* GEMM_RELU_FAMILY_* */
    int32_t reserved[4];     /* zero */
} gemm_relu_tile_desc;

/*
 * Fills *desc for a tile id < gemm_relu_tile_count(). Returns GEMM_RELU_EINVAL
 * for a NULL desc and GEMM_RELU_EUNSUPPORTED for an unknown id (desc is then
 * left untouched). Host-only; makes no HIP call.
 */
int gemm_relu_tile_info(int tile, gemm_relu_tile_desc* desc);

/*
 * The block order and group size a launch of `tile` over an M x N output
 * uses when opts leave both at their defaults (block_order
 * GEMM_RELU_ORDER_DEFAULT, group_m 0), as chosen for the grid of tiles that
 * the TileLang example's block-order swizzle (section "Escribamos un GEMM")
 * walks: *block_order gets GEMM_RELU_ORDER_DEFAULT (grouped) or
 * GEMM_RELU_ORDER_ROW_MAJOR, *group_m the tile-rows per group of the grouped
 * order. Returns GEMM_RELU_EINVAL for a NULL pointer or a negative size and
 * GEMM_RELU_EUNSUPPORTED for an unknown tile (outputs then left untouched).
 * Host-only; makes no HIP call.
 */
int gemm_relu_default_order(int tile, int64_t M, int64_t N, int32_t* block_order, int32_t* group_m);

/*
 * Transposed operands: the transpose_A / transpose_B flags of the tile-level
 * product in the same TileLang example (the notes under the program in
 * "Escribamos un GEMM"). C = epilogue(op(A) @ op(B)), where
 *   op_a = GEMM_RELU_OP_N: A is M x K as stored (row-major, leading dim K);
 *   op_a = GEMM_RELU_OP_T: A is stored K x M (leading dim M) and op(A) is its
 *                          transpose;
 *   op_b = GEMM_RELU_OP_N: B is K x N as stored (leading dim N);
 *   op_b = GEMM_RELU_OP_T: B is stored N x K (leading dim K) and op(B) is its
 *                          transpose.
 * C is always M x N row-major (leading dim N). Everything else -- sizes,
 * accumulation, epilogue, rounding, ownership, errors -- is as for the
 * untransposed calls; an op value other than N or T gives GEMM_RELU_EINVAL.
 * The vector kernels need the leading dimensions of A (K or M), B (N or K)
 * and C (N) to be multiples of 8 and 16-byte aligned pointers; other shapes
 * take the element-wise path.
 */
#define GEMM_RELU_OP_N 0
#define GEMM_RELU_OP_T 1

/* C = ReLU(op(A) @ op(B)); opts as for gemm_relu_f16_ex (may be NULL). */
int gemm_relu_f16_op(int64_t M, int64_t N, int64_t K, const void* A, int op_a, const void* B, int op_b,
                     void* C, void* stream, const gemm_relu_opts* opts);

/* C = GELU(op(A) @ op(B) + bias); bias and opts as for gemm_bias_gelu_f16_ex. */
int gemm_bias_gelu_f16_op(int64_t M, int64_t N, int64_t K, const void* A, int op_a, const void* B, int op_b,
                          const void* bias, void* C, void* stream, const gemm_relu_opts* opts);

/*
 * The tile the library would use for this problem without opts, or -1 for the
 * generic element-wise path that serves shapes whose K or N is not a multiple
 * of 8 or whose pointers are not 16-byte aligned (pass NULL pointers to ask
 * about shapes alone). Host-only; makes no HIP call.
 */
int gemm_relu_select_tile(int64_t M, int64_t N, int64_t K,
                          const void* A, const void* B, const void* C);

/* Same, for operand layouts op_a and op_b (-1 also for an invalid op). */
int gemm_relu_select_tile_op(int64_t M, int64_t N, int64_t K, int op_a, int op_b,
                             const void* A, const void* B, const void* C);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_RELU_H */
