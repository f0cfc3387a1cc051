/*
 * mm.h -- C ABI of the MI355X (gfx950) quantized skinny MUL_MAT library.
 *
 * The library computes the ggml-style MUL_MAT at LLM-decode shapes,
 *
 *     dst[M x N] = src1[M x K] . src0[N x K]^T        (row-major, contiguous)
 *
 * for the three kinds named in llama.cpp PR 1632 "mulmat tune", Introduction:
 * F32 x F32, F16 x F32 and quantized (here Q4_0) x F32.  For the quantized
 * kind, src1 is first quantized to Q8_0 (the INIT stage of that page; the
 * "wdata" buffer of the Arm China NUMA article, MulMat operator section) and
 * the product is taken between the Q4_0 weights and that Q8_0 copy.
 *
 * Block formats (not printed on the pages, which only name the types; the
 * library is specified against the ggml layouts):
 *   Q4_0: 18 bytes per 32 values: fp16 d (little endian), then 16 bytes;
 *         byte i holds code q[i] in its low nibble and q[i+16] in its high
 *         nibble; value = d * (q - 8).
 *         d = (signed absmax) / -8, q = clamp(floor(x/d + 8.5), 0, 15).
 *   Q8_0: 34 bytes per 32 values: fp16 d, then 32 int8 codes; value = d * q.
 *         d = absmax / 127, q = round(x/d) (half away from zero).
 *   In both, x/d is evaluated as x * (1/d) with one correctly rounded fp32
 *   reciprocal per block, codes come from the fp32 d, and only the stored d
 *   is rounded to fp16 (round to nearest even).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc / torch CUDA
 *     memory).  Sizes are element counts.  Calls are asynchronous on
 *     `stream` (a hipStream_t; NULL = the null stream) and never synchronise.
 *   - The caller owns every buffer, including the workspace `ws`; the
 *     library allocates no device memory and keeps no per-call state.  Calls
 *     on different streams may run concurrently if their buffers differ.
 *   - Arguments are validated on the host before any HIP call; on error the
 *     function returns a negative mm_status and launches nothing.
 *   - dst is overwritten (never accumulated into).  M == 0 or N == 0 is a
 *     no-op; K == 0 writes zeros (the empty sum).
 *   - Results are deterministic run to run: there are no floating-point
 *     atomics; split-K partial sums are added in a fixed order.
 */
#ifndef QSG_MM_H
#define QSG_MM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mm_status {
    MM_OK = 0,
    MM_ERR_NULL = -1,      /* a required pointer is NULL                         */
    MM_ERR_SHAPE = -2,     /* negative size, K % 32 != 0 for a block type, or a size too large */
    MM_ERR_ALIGN = -3,     /* pointer not aligned as documented per entry point  */
    MM_ERR_WORKSPACE = -4, /* ws_bytes smaller than mm_mul_mat_workspace_size()  */
    MM_ERR_ALIAS = -5,     /* dst (or ws) overlaps an input, or ws overlaps dst  */
    MM_ERR_DEVICE = -6,    /* current device is not gfx950                       */
    MM_ERR_HIP = -7,       /* a HIP runtime call or launch failed                */
    MM_ERR_ARG = -8        /* unknown type or variant                            */
} mm_status;

typedef enum mm_type {
    MM_TYPE_F32 = 0,
    MM_TYPE_F16 = 1,
    MM_TYPE_Q4_0 = 2,
    MM_TYPE_Q8_0 = 3,
    MM_TYPE_Q4_0R = 4      /* Q4_0 weights in the repacked layout (mm_repack_q4_0) */
} mm_type;

/*
 * mm_quantize_q4_0 -- x[nrows][k] (f32) -> y[nrows][k/32] Q4_0 blocks (18 B each).
 * Weight quantisation (setup, outside the decode loop): src0 of the
 * quantized MUL_MAT kind arrives as one of the block types the mulmat tune
 * PR lists in its Introduction (Q4_0 among them; its Results section names
 * Q4_0, Q5_0 and Q8_0); the encoding is the Q4_0 one above.  k % 32 == 0.
 * x must be 16-byte aligned; y needs 2-byte alignment.  y must not overlap
 * x.
 */
mm_status mm_quantize_q4_0(const float* x, void* y, int64_t nrows, int64_t k, void* stream);

/*
 * mm_quantize_q8_0 -- x[nrows][k] (f32) -> y[nrows][k/32] Q8_0 blocks (34 B each).
 * The activation quantisation that the Q4_0 product applies to src1 (the
 * INIT stage / wdata): its bytes are identical to the Q8_0 content
 * mm_mul_mat_q4_0_f32 computes internally.  k % 32 == 0.  x 16-byte aligned,
 * y 2-byte aligned, no overlap.
 */
mm_status mm_quantize_q8_0(const float* x, void* y, int64_t nrows, int64_t k, void* stream);

/*
 * mm_mul_mat_q4_0_f32 -- dst[M][N] (f32) = Q8_0(src1)[M][K] . Q4_0 src0[N][K]^T.
 *   src0: N rows of K/32 Q4_0 blocks (row pitch 18*K/32 bytes), 2-byte aligned
 *         (4-byte alignment and an even K/32 select the fast load path).
 *   src1: f32 [M][K], 16-byte aligned.  dst: f32 [M][N], 4-byte aligned.
 *   K % 32 == 0.
 *   ws:   workspace of at least mm_mul_mat_workspace_size(MM_TYPE_Q4_0, M, N, K)
 *         bytes, 256-byte aligned; holds the Q8_0 wdata and any split-K
 *         partial sums.  Its content on entry is irrelevant.
 * dst[m][n] = sum_b f32(d_w[n][b]) * f32(d_a[m][b]) * S_b[m][n], with the
 * int32 block dot S_b = sum_j (q4 - 8) * q8, accumulated in fp32.
 */
mm_status mm_mul_mat_q4_0_f32(const void* src0, const float* src1, float* dst,
                              int64_t M, int64_t N, int64_t K,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * mm_mul_mat_q4_0_f32_noalloc -- mm_mul_mat_q4_0_f32 without a caller
 * workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 *   Same operands, layouts, alignment rules, result and determinism as
 *   mm_mul_mat_q4_0_f32 (same kernels; the output is bit-identical).  The
 *   workspace is a fixed array of 64 MiB (67108864 bytes) in device memory
 *   that the library holds on each GPU it runs on until the process ends;
 *   the call itself allocates nothing.  A shape whose
 *   mm_mul_mat_workspace_size(MM_TYPE_Q4_0, M, N, K) exceeds 64 MiB returns
 *   MM_ERR_WORKSPACE before any HIP call (e.g. M = 512 fits for every N up
 *   to 128256 at K = 4096).  Every call on one GPU shares that GPU's array:
 *   calls that may overlap in time on one GPU (different streams, or
 *   different host threads) race and must be serialised by the caller.
 */
mm_status mm_mul_mat_q4_0_f32_noalloc(const void* src0, const float* src1, float* dst,
                                      int64_t M, int64_t N, int64_t K, void* stream);

/*
 * The two stages of mm_mul_mat_q4_0_f32, exposed separately (llama.cpp PR
 * 1632 "mulmat tune", Introduction: the quantized kind runs an INIT stage
 * that converts src1, then the COMPUTE stage).  mm_mul_mat_q4_0_f32 is
 * exactly mm_q4_0_init followed by mm_q4_0_compute on the same stream.
 *
 * mm_q4_0_init: quantizes src1 f32 [M][K] (16-byte aligned) to Q8_0 into the
 *   workspace (layout private to the library; the content equals
 *   mm_quantize_q8_0 of src1) and prepares the split-K state.  ws as for
 *   mm_mul_mat_q4_0_f32 with the same (M, N, K).
 * mm_q4_0_compute: dst[M][N] = wdata . src0^T from a workspace that an
 *   mm_q4_0_init with the SAME (M, N, K) filled earlier on this stream (or
 *   that a completed mm_q4_0_compute left behind: compute leaves the wdata
 *   unchanged).  One init can thus serve several src0 of the same shape
 *   (e.g. the q, k and v projections of one activation).  Calls that share a
 *   workspace must not overlap in time.
 */
mm_status mm_q4_0_init(const float* src1, void* ws, int64_t M, int64_t N, int64_t K,
                       size_t ws_bytes, void* stream);
mm_status mm_q4_0_compute(const void* src0, float* dst, int64_t M, int64_t N, int64_t K,
                          const void* ws, size_t ws_bytes, void* stream);

/*
 * mm_mul_mat_q4_0_f32_group -- several Q4_0 products that share src1, in as
 * few launches as possible: dsts[i][M][Ns[i]] = Q8_0(src1) . src0s[i]^T for
 * i < count (1 <= count <= 8), e.g. the q, k and v projections of one
 * activation, or the ffn gate and up projections.  src0s, dsts and Ns are
 * HOST arrays of count entries; every src0s[i] and dsts[i] follows the rules
 * of mm_mul_mat_q4_0_f32 (shared M, K, src1); the dsts must not overlap
 * each other or any src0.  Results equal count separate mm_mul_mat_q4_0_f32
 * calls.  ws: mm_mul_mat_q4_0_group_workspace_size(count, Ns, M, K) bytes.
 */
mm_status mm_mul_mat_q4_0_f32_group(int count, const void* const* src0s, float* const* dsts,
                                    const int64_t* Ns, const float* src1, int64_t M, int64_t K,
                                    void* ws, size_t ws_bytes, void* stream);
size_t mm_mul_mat_q4_0_group_workspace_size(int count, const int64_t* Ns, int64_t M, int64_t K);

/*
 * Weight repack at load time (DeepSpeed-Inference reading notes, III.C
 * SBI-GeMM, item 3: the weights are laid out once, at initialisation, so
 * that every thread of the product reads whole cache lines of what it
 * consumes).  The repacked layout ("Q4_0R") holds the same 18 bytes per
 * block, grouped per tile of 16 weight rows and phase of 8 blocks (256
 * values of K) into 2304-byte chunks, tile-major ([ceil(N/16)][ceil(K/256)]):
 *   bytes    0..2047: codes, [half hh][lane l][4 dwords]: lane l = i + 16 g
 *                     holds code bytes 4g..4g+3 of row i of the tile for
 *                     blocks 4 hh + 0..3 (low nibbles: elements 4g..4g+3,
 *                     high nibbles: elements 16+4g..19+4g);
 *   bytes 2048..2303: scales, [row i][block b] binary16 d.
 * Rows past N and blocks past K/32 are padding (codes 0x88, scale 0).
 *
 * mm_repacked_q4_0_bytes -- size of the repacked form of N x K Q4_0 weights
 *   (ceil(N/16) * ceil(K/256) * 2304); -1 if K % 32 != 0 or a size is
 *   negative.  Pure host function.
 * mm_repack_q4_0 -- src0 (Q4_0 [N][K/32] blocks, 2-byte aligned) -> dst
 *   (repacked, 16-byte aligned, mm_repacked_q4_0_bytes(N, K) bytes, all
 *   written including padding).  Buffers must not overlap.
 * mm_unpack_q4_0 -- the inverse: repacked src (16-byte aligned) -> Q4_0
 *   [N][K/32] blocks in dst (2-byte aligned); unpack(repack(w)) == w byte
 *   for byte.
 * mm_mul_mat_q4_0r_f32 -- mm_mul_mat_q4_0_f32 with src0 in the repacked
 *   layout (16-byte aligned): the same result (block dots bit-exact,
 *   dst within the same bound; the kernels differ, so dst may differ from
 *   the plain call in the last bits).  ws:
 *   mm_mul_mat_workspace_size(MM_TYPE_Q4_0R, M, N, K) bytes.
 * Errors as for the other entry points (MM_ERR_SHAPE for K % 32 != 0).
 */
int64_t mm_repacked_q4_0_bytes(int64_t N, int64_t K);
mm_status mm_repack_q4_0(const void* src0, void* dst, int64_t N, int64_t K, void* stream);
mm_status mm_unpack_q4_0(const void* src0r, void* dst, int64_t N, int64_t K, void* stream);
mm_status mm_mul_mat_q4_0r_f32(const void* src0r, const float* src1, float* dst,
                               int64_t M, int64_t N, int64_t K,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * mm_mul_mat_q8_0_f32 -- dst[M][N] (f32) = Q8_0(src1)[M][K] . Q8_0 src0[N][K]^T.
 * The quantized kind with Q8_0 weights: llama.cpp PR 1632 "mulmat tune"
 * names Q8_0 among the quantized src0 types it measures (Results section);
 * its blocks are the Q8_0 blocks above, the same ones the INIT stage writes
 * for src1 (mm_quantize_q8_0 makes them from f32 weights).
 *   src0: N rows of K/32 Q8_0 blocks (row pitch 34*K/32 bytes), 4-byte
 *         aligned.  src1: f32 [M][K], 16-byte aligned.  dst: f32 [M][N],
 *         4-byte aligned.  K % 32 == 0.
 *   ws:   mm_mul_mat_workspace_size(MM_TYPE_Q8_0, M, N, K) bytes, 256-byte
 *         aligned (the Q8_0 copy of src1 and any split-K partial sums).
 * dst[m][n] = sum_b f32(d_w[n][b]) * f32(d_a[m][b]) * S_b[m][n], with the
 * int32 block dot S_b = sum_j qw * qa of the two signed code sets (|S_b| <=
 * 32 * 128 * 128), accumulated in fp32.  M <= 2 with K a multiple of 64:
 * one kernel that quantizes src1 itself; 2 < M <= 32 with K a multiple
 * of 64: INIT, then the skinny int8 MFMA kernel (16 weight rows per
 * workgroup, passes of 8, 16 or 32 src1 rows); otherwise INIT, then the
 * tiled int8 MFMA kernel.
 */
mm_status mm_mul_mat_q8_0_f32(const void* src0, const float* src1, float* dst,
                              int64_t M, int64_t N, int64_t K,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * mm_mul_mat_f16_f32 -- dst[M][N] = src1[M][K] . f32(src0[N][K])^T, fp32 accumulation.
 * The F16 x F32 kind of llama.cpp PR 1632 "mulmat tune", Introduction
 * (src0 F16, src1 and dst F32; no INIT stage).
 *   src0: IEEE binary16 [N][K], 2-byte aligned.  src1: f32 [M][K], 4-byte
 *   aligned.  dst: f32, 4-byte aligned.  Any K >= 0.
 *   Precision follows the kernel mm_dispatch reports for the shape.
 *   Narrow kernel (M = 1, and small M where the dispatch table picks it;
 *   any M up to the wide kernel's whose operands are not 16-byte aligned
 *   or whose K is not a multiple of 8 or exceeds 2^23): fp32 FMA of src1
 *   as given and the widened weights.
 *   Skinny kernel (built-in rules: 2 <= M <= 16, and up to 64 with at most
 *   8192 weight rows; the measured table gives it, e.g., 4096 x 4096 up to
 *   45 rows): the same exact fp32 products on the fp32 matrix cores.  Both
 *   hold for every finite src1 in the fp32 range.  Wide kernel (larger M,
 *   and on the shapes where the table measured it faster, e.g. 14336 x 4096
 *   from M = 3): src1 is rounded to binary16 for the fp16 matrix cores after
 *   scaling each row by a power of two that puts its largest magnitude in
 *   [2^14, 2^15) (undone exactly on the outputs), so every row keeps 11
 *   significant bits whatever its magnitude (row-normwise effect about
 *   1e-4; only elements below 2^-28 of their row's largest magnitude lose
 *   bits, a contribution far under the bound).  All inside the 1e-3
 *   row-normwise bound of this kind.
 *   ws: mm_mul_mat_workspace_size(MM_TYPE_F16, ...) bytes (0 when that is
 *   0); for the larger M it holds src1 as binary16 and the row exponents.
 */
mm_status mm_mul_mat_f16_f32(const uint16_t* src0, const float* src1, float* dst,
                             int64_t M, int64_t N, int64_t K,
                             void* ws, size_t ws_bytes, void* stream);

/*
 * mm_mul_mat_f32 -- dst[M][N] = src1[M][K] . src0[N][K]^T, all f32 products,
 *   fp32 accumulation.  The F32 x F32 kind of llama.cpp PR 1632 "mulmat
 *   tune", Introduction.  Vector FMA at M = 1; from M = 2 the fp32 MFMA when
 *   src0 and src1 are 16-byte aligned and K is a multiple of 4 of at most
 *   2^23 (else the vector kernel).  All pointers 4-byte aligned.  Any K >= 0.
 *   ws: mm_mul_mat_workspace_size(MM_TYPE_F32, ...) bytes (0 at every shape
 *   today; pass it anyway).
 */
mm_status mm_mul_mat_f32(const float* src0, const float* src1, float* dst,
                         int64_t M, int64_t N, int64_t K,
                         void* ws, size_t ws_bytes, void* stream);

/* Bytes of workspace the product of `type` (F32, F16, Q4_0, Q8_0 or Q4_0R)
 * needs at this shape; 0 for an invalid shape or type.  Pure host function. */
size_t mm_mul_mat_workspace_size(int type, int64_t M, int64_t N, int64_t K);

/* Bytes of one row of K values of `type`; -1 if K is invalid for it. */
int64_t mm_row_bytes(int type, int64_t K);

/* Static description of a status code.  Never NULL. */
const char* mm_status_string(int status);

/*
 * mm_dispatch -- the kernel choice mm_mul_mat_* makes at this shape (pure
 * host function).  Writes 5 ints to out (may be NULL):
 *   out[0] variant: 1 = narrow-M kernel, 2 = wide-M (MFMA) kernel (Q4_0,
 *          F16), 3 = skinny MFMA kernel (a few src1 rows; F32 from 2)
 *   out[1] split-K factor (1 = none)
 *   out[2] rows of src1 per pass (narrow, skinny) or output tile rows (wide)
 *   out[3] output tile columns (wide), src0 rows per wave (narrow) or
 *          waves per workgroup (skinny)
 *   out[4] kernels one call launches on the stream (for Q4_0 at small M
 *          the INIT stage is fused into the product kernel: 1; the wide F16
 *          kernel adds its src1 pre-pass, a K split the reduce)
 * Returns MM_OK or MM_ERR_SHAPE / MM_ERR_ARG.
 */
mm_status mm_dispatch(int type, int64_t M, int64_t N, int64_t K, int* out);

/*
 * mm_debug_mul_mat -- test entry: the same product as mm_mul_mat_<type>,
 * with the kernel forced (variant 0 = as dispatched, 1 = narrow, 2 = wide
 * (Q4_0, Q4_0R, Q8_0 and F16), 3 = skinny MFMA (not Q8_0);
 * MM_ERR_ARG for a variant the type does not have; MM_ERR_SHAPE for the
 * narrow or skinny kernel of a block type forced on more than 65535 src1
 * rows, which those kernels' grids cannot hold: mm_mul_mat_* takes the
 * wide kernel there, and F16 / F32 run such products as several launches
 * over consecutive row ranges)
 * and, for Q4_0 and Q4_0R, the int32 block dots S_b[m][n][b] of output
 * columns n0 <= n < n1 also written to `dots` ([M][n1-n0][K/32] int32, may
 * be NULL) by the production kernel itself; for Q8_0 by the wide kernel
 * only (MM_ERR_ARG when the call would take the fused narrow kernel).
 * Workspace: mm_debug_workspace_size().
 */
mm_status mm_debug_mul_mat(int type, const void* src0, const float* src1, float* dst,
                           int32_t* dots, int64_t M, int64_t N, int64_t K,
                           int64_t n0, int64_t n1, int variant,
                           void* ws, size_t ws_bytes, void* stream);

size_t mm_debug_workspace_size(int type, int64_t M, int64_t N, int64_t K, int variant);

#ifdef __cplusplus
}
#endif

#endif /* QSG_MM_H */
