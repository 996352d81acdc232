/*
 * gbb -- fused dequantize-and-multiply GEMV/GEMM over weight-only quantized
 * LLM layers, for AMD Instinct MI355X (gfx950).
 *
 * Two weight formats:
 *
 *  1. Block format.  The weight matrix W [N out][K in] is cut into blocks of
 *     64 output rows x 128 input columns; every block has one bitwidth
 *     b in {1,2,3,4,6,8} ("ScaleBITS: Scalable Bitwidth Search for
 *     Hardware-Aligned Mixed-Precision LLMs", explainer page, section 1.2.2
 *     "hardware-aligned block partition" and section 4.2 for the bitwidth set).
 *     Each (row, 128-column group) has an fp16 scale s and zero z; codes are
 *     q = clamp(rint(w / s) + z, 0, 2^b - 1) and dequantize as (q - z) * s
 *     ("MixLLM: LLM Quantization with Global Mixed-precision between
 *     Output-features and Highly-efficient System Design", section 2.1).
 *
 *  2. Output-feature mixed format ("W4.4A8", MixLLM page, sections 3.1.1 and
 *     3.3): a set of salient output rows is quantized 8-bit symmetric, the
 *     other rows 4-bit asymmetric, both with group 128, and multiplied with
 *     8-bit symmetric activations by a two-step dequantization: an integer
 *     product per group, then the two scales.
 *
 * Conventions for every entry point:
 *  - Matrices are row-major.  fp16 values are passed as their 16-bit patterns
 *    (uint16_t).  y = x . W^T: x is [M][K], y is [M][N].
 *  - "host" pointers are CPU memory; "device" pointers are GPU memory of the
 *    current HIP device (hipMalloc or a torch tensor).  The caller owns every
 *    buffer.  `stream` is a hipStream_t (NULL = the default stream).
 *  - Device entry points only validate arguments and enqueue kernels on
 *    `stream`; they never allocate, never synchronize and return before the
 *    work finishes.  Faults inside kernels are not reported by the call.
 *  - Nothing throws, aborts or prints.  A negative status is an error; the
 *    text of the last error of the calling thread is gbb_last_error().
 *  - Device pointers must be 16-byte aligned; x and y must not overlap.
 */
#ifndef GBB_H
#define GBB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int gbb_status;

enum {
  GBB_OK = 0,
  GBB_E_ARG = -1,     /* null pointer, non-positive size, bad flag or option */
  GBB_E_SHAPE = -2,   /* N % 64 != 0 or K % 128 != 0 (block format), or bad row set */
  GBB_E_BITS = -3,    /* a bitwidth outside {1,2,3,4,6,8}, or a bad given zero */
  GBB_E_ALIGN = -4,   /* a device pointer that is not 16-byte aligned */
  GBB_E_SPACE = -5,   /* an output or workspace capacity that is too small */
  GBB_E_FORMAT = -6,  /* an image header that does not match the arguments */
  GBB_E_DEVICE = -7   /* a HIP runtime or launch error */
};

/* Text of the last non-OK status returned to this thread ("" if none). */
const char* gbb_last_error(void);

/* Library version: 10000 * major + 100 * minor + patch. */
int gbb_version(void);

/* ======================================================================== */
/* Block format                                                             */
/* ======================================================================== */

/* Byte size of the packed image for an N x K matrix with the per-block
 * bitwidth map `bits` (host, uint8 [N/64][K/128], block-row major): the
 * block-wise storage with a small per-block bitwidth record of the ScaleBITS
 * explainer page, section 3.2, in the layout of layout.h.  The size
 * is a 64-byte header, then 256-byte aligned sections: one byte per block,
 * 4 * (blocks + 1) bytes of offsets, 256 bytes of scale/zero per block and
 * 64 * 128 * b / 8 = 1024 * b bytes of codes per block.  Returns 0 on a bad
 * argument (see gbb_last_error). */
size_t gbb_packed_bytes(const uint8_t* bits, int N, int K);

#define GBB_PACK_GIVEN_SZ 1u  /* use the caller's scale/zero instead of min/max */

/* Quantize and pack (host, synchronous, deterministic; may use several CPU
 * threads).
 *   W      host fp16 [N][K].
 *   bits   host uint8 [N/64][K/128], each in {1,2,3,4,6,8}.
 *   scale, zero  host fp16 [N][K/128].  Without GBB_PACK_GIVEN_SZ they are
 *          outputs (may be NULL): per (row, group) s = fp16((max - min) /
 *          (2^b - 1)) and z = clamp(rint(-min / s), 0, 2^b - 1), decisions in
 *          fp64, round-half-even (MixLLM page, section 2.1, with min/max
 *          ranges).  With GBB_PACK_GIVEN_SZ they are inputs (e.g. scales from
 *          a clipping search): s must be finite and > 0, z an integer in
 *          [0, 2^b - 1].
 *   image  host output of gbb_packed_bytes(bits, N, K) bytes (image_cap).
 * Codes q = clamp(rint(w / s) + z, 0, 2^b - 1).  The image can be copied to
 * the device as is and shared by any number of streams. */
gbb_status gbb_pack_blocks(const uint16_t* W, int N, int K, const uint8_t* bits,
                           uint16_t* scale, uint16_t* zero, unsigned flags,
                           void* image, size_t image_cap);

/* Offline bitwidth allocation (host, synchronous, deterministic): one
 * bitwidth from {1,2,3,4,6,8} per 64x128 block with a mean of at most
 * target_bits, by the batched greedy of the ScaleBITS explainer page
 * (section 2.2: gamma * nblk blocks per round, gamma = 0.05 there; section
 * 4.2: the bitwidth set and the 3-bit start).  The pages' gradient
 * sensitivity needs a model and calibration data; here block i's cost at
 * bitwidth b is S_i * e_i(b), S_i = sum |w| over the block, e_i(b) = sum
 * (w - w')^2 under gbb_pack_blocks' quantizer.  Rounds lower the cheapest
 * blocks while over budget, raise the most beneficial ones that fit while
 * under it, then trade the most beneficial raises for the cheapest
 * lowerings that pay for them while that lowers the summed cost; ties go to
 * the lower block index.
 *   W            fp16 [N][K], finite; N % 64 == 0, K % 128 == 0.
 *   target_bits  mean bitwidth budget in [1, 8].
 *   gamma        fraction of the blocks moved per round, in (0, 1].
 *   bits         host output [N/64][K/128], row-major.
 * Errors: GBB_E_ARG (NULL, non-finite W, target or gamma out of range),
 * GBB_E_SHAPE. */
gbb_status gbb_allocate_bits(const uint16_t* W, int N, int K, double target_bits, double gamma,
                             uint8_t* bits);

/* Bidirectional channel reordering (ScaleBITS explainer page, section
 * 1.2.1) with |W| as the sensitivity: rows and columns by descending L1
 * norm (exact), ties to the lower index.  Packing W[row_order][:, col_order]
 * gathers the large weights in the top-left blocks; the caller permutes the
 * activations (x[:, col_order]) and un-permutes the outputs accordingly.
 *   W          fp16 [N][K], finite, any N, K > 0.
 *   row_order  host output [N] (a permutation of 0 ... N-1).
 *   col_order  host output [K].
 * Errors: GBB_E_ARG. */
gbb_status gbb_channel_order(const uint16_t* W, int N, int K, int32_t* row_order, int32_t* col_order);

/* Check a host copy of an image header against N and K (GBB_E_FORMAT): the
 * block-wise storage of the ScaleBITS explainer page, section 3.2 (version 1,
 * 64x128 blocks) or its 64x64 variant of section 4.2 (version 2). */
gbb_status gbb_check_image(const void* image, size_t image_bytes, int N, int K);

/* Workspace bytes gbb_gemm_mixed_w needs for (N, K, M) (the fused product of
 * the ScaleBITS explainer page, section 3.2, when its K range is split over
 * workgroups); may be 0.  On the decode route, when K is split across
 * workgroups, it is M * N * 12 (per output element an int64 fixed-point and
 * an fp32 accumulator), or for 17 <= M <= 32 on matrices of at least 2^26
 * weights (two block rows per workgroup) fp32 partials, segments * M * N * 4
 * bytes, summed in segment order by a second launch; for batches run as
 * 32-token chunks, that of the largest chunk; a smaller workspace is an
 * error.  On the prefill route it is
 * the fp32 partials of the K split described under
 * gbb_gemm_mixed_w_path_workspace, and a smaller workspace only shortens the
 * split.  The workspace must be zero-filled once before its first use; every
 * call leaves it zero-filled again.  Calls that run at the same time need
 * separate workspaces. */
size_t gbb_gemm_mixed_w_workspace(int N, int K, int M);
/* The same for gbb_gemm_mixed_w_path with a given path (0 equals
 * gbb_gemm_mixed_w_workspace).  For the prefill kernel (path 2, or path 0
 * when it takes the batch) the workspace holds the K split: when the tile
 * grid of 128 tokens x 512 rows fills at most half of the compute units,
 * each tile's K range is cut into up to 16 segments of at least 1024
 * columns, whose fp32 partials live in the workspace (segments * M * N * 4
 * bytes) until a second launch of the same call adds them in segment order
 * and clears them.  A prefill call whose
 * workspace is smaller (or NULL) takes as many segments as fit, down to
 * none; it never fails for lack of workspace. */
size_t gbb_gemm_mixed_w_path_workspace(int N, int K, int M, int path);

/* y = x . dequant(W)^T over a packed block image (ScaleBITS explainer page,
 * section 3.2: the weight is dequantized inside the matrix product, one
 * bitwidth per 64x128 block).
 *   image  device copy of gbb_pack_blocks' output for this N, K.
 *   x      device fp16 [M][K];  y device fp16 [M][N] (fp32 accumulation,
 *          round-to-nearest-even at the end).
 *   M >= 1.  M <= 32 runs the decode kernels (weights streamed once, matrix
 *   cores for the dot products).  Larger M runs the tiled prefill kernel,
 *   with its K range split into segments when its grid of 128-token x
 *   512-row tiles is small (see gbb_gemm_mixed_w_path_workspace), or the
 *   decode kernels in 32-token chunks, one launch each, when the chunks are
 *   few against the prefill grid: chunks x max(CUs / 4, split prefill
 *   workgroups) <= 3/4 of the device's compute units, a ragged last chunk
 *   counted as half.
 *   workspace/ws_bytes  device memory of gbb_gemm_mixed_w_workspace(N, K, M)
 *          bytes (NULL allowed when that is 0).  On the prefill route the
 *          number of K segments follows ws_bytes, and with it the order of
 *          the fp32 sums: for one ws_bytes the result is the same on every
 *          call, across sizes it may differ in the last bits.
 * Errors: GBB_E_ARG (NULL image/x/y, N or K <= 0, M < 0, x and y overlap,
 * missing workspace), GBB_E_SHAPE (N % 64, K % 128, N or K above 2^20, or
 * M * K >= 2^31 on the prefill kernel), GBB_E_ALIGN, GBB_E_SPACE (workspace
 * too small), GBB_E_DEVICE (launch failed).  M == 0 does nothing. */
gbb_status gbb_gemm_mixed_w(const void* image, int N, int K, const uint16_t* x,
                            uint16_t* y, int M, void* workspace, size_t ws_bytes,
                            void* stream);

/* Allocation-free variant of gbb_gemm_mixed_w, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments (without the workspace),
 * checks and kernels as gbb_gemm_mixed_w; the split-K accumulators live in a
 * fixed array of GBB_NOALLOC_SCRATCH_BYTES of device memory that the library
 * holds on each GPU it runs on, from the first call on that GPU until the
 * process ends.  That first call also zero-fills the array on `stream`
 * (again on later calls while the fills so far were recorded under stream
 * capture); every call leaves it zero.  All calls on one GPU share that
 * GPU's array, so calls that may overlap on one GPU (several streams or
 * threads, graphs replayed concurrently) race and give wrong results.  The
 * call allocates and frees nothing.
 * The prefill route's K split takes as many segments as the array holds, so
 * the result equals gbb_gemm_mixed_w's with ws_bytes =
 * GBB_NOALLOC_SCRATCH_BYTES.
 * Errors: those of gbb_gemm_mixed_w; GBB_E_SPACE when the decode route
 * needs more than GBB_NOALLOC_SCRATCH_BYTES of workspace (no shape the block
 * entry points accept needs more than 12 MiB);
 * GBB_E_DEVICE when the array's address cannot be obtained. */
#define GBB_NOALLOC_SCRATCH_BYTES (16u << 20)
gbb_status gbb_gemm_mixed_w_noalloc(const void* image, int N, int K, const uint16_t* x,
                                    uint16_t* y, int M, void* stream);

/* Grouped products: n (1 ... 32) independent block GEMMs y[i] = x[i] .
 * dequant(W_i)^T with one M, for products that do not depend on each other
 * (the concurrent sub-problems of the MixLLM page, section 3.3; the
 * per-bitwidth execution plan of the ScaleBITS explainer page, section 3.2).
 * For M <= 16 all of them run as ONE launch of the decode kernels: problem
 * i's workgroups follow problem i-1's in a single grid, so small products
 * share the GPU instead of paying a launch and a ramp each.  For larger M
 * the problems run one after another, as gbb_gemm_mixed_w runs them.
 *   images[i]  device image of N[i] x K[i] (gbb_pack_blocks).
 *   x[i], y[i] device fp16 [M][K[i]] and [M][N[i]]; no y may overlap another
 *              problem's x or y.
 *   workspace  device memory of gbb_gemm_mixed_w_batched_workspace(n, N, K,
 *              M) bytes (NULL allowed when that is 0), zero-filled once
 *              before first use; every call leaves it zero-filled.
 * Errors: GBB_E_ARG (n outside 1 ... 32, NULL arrays, missing workspace),
 * those of gbb_gemm_mixed_w for each problem (with its index in the
 * message), GBB_E_SPACE, GBB_E_DEVICE. */
size_t gbb_gemm_mixed_w_batched_workspace(int n, const int* N, const int* K, int M);
gbb_status gbb_gemm_mixed_w_batched(int n, const void* const* images, const int* N, const int* K,
                                    const uint16_t* const* x, uint16_t* const* y, int M,
                                    void* workspace, size_t ws_bytes, void* stream);

/* Whole-layer execution (ScaleBITS explainer page, section 3.2: an execution
 * plan generated for a given bit configuration; MixLLM page, section 3.3:
 * the kernels of a step replayed from a captured graph).  Captures n
 * gbb_gemm_mixed_w calls, in order, into one HIP graph: call i multiplies
 * x[i] (device fp16 [M][K[i]]) by images[i] (device, N[i] x K[i]) into y[i]
 * (device fp16 [M][N[i]]).  Every pointer is recorded as is and must stay
 * valid, with the same shapes, for the graph's life; each call is checked as
 * gbb_gemm_mixed_w checks it, and the first failing call's status is
 * returned.  The calls share one workspace (device, zero-filled once before
 * the first launch, ws_bytes >= the largest gbb_gemm_mixed_w_workspace of
 * the calls); they run one after the other and leave it zero-filled, so
 * launches of the graph on one stream may follow each other, but launches
 * that may run at the same time need graphs with separate workspaces.  Host
 * call; captures on a stream of its own (default priority), allocates only
 * the graph.  On success *out owns the graph.
 * Errors: GBB_E_ARG (NULL, n < 1, M < 1), those of gbb_gemm_mixed_w,
 * GBB_E_DEVICE (capture or instantiation failed). */
typedef struct gbb_graph gbb_graph;
gbb_status gbb_graph_create(int n, const void* const* images, const int* N, const int* K,
                            const uint16_t* const* x, uint16_t* const* y, int M,
                            void* workspace, size_t ws_bytes, gbb_graph** out);

/* Launch a captured graph on `stream` (asynchronous). */
gbb_status gbb_graph_launch(const gbb_graph* g, void* stream);

/* Free a graph (NULL is allowed).  The caller makes sure no launch of it is
 * still running. */
gbb_status gbb_graph_destroy(gbb_graph* g);

/* Same as gbb_gemm_mixed_w with the kernel chosen by `path`: 0 = automatic,
 * 1 = decode kernel (requires M <= 32), 2 = prefill kernel.  For tests. */
gbb_status gbb_gemm_mixed_w_path(const void* image, int N, int K, const uint16_t* x,
                                 uint16_t* y, int M, void* workspace, size_t ws_bytes,
                                 int path, void* stream);

/* Debug exports over a device image, for bit-exactness tests.
 *   gbb_unpack_codes: q device uint8 [N][K], the codes read back from the
 *   block-wise storage (ScaleBITS explainer page, section 3.2).
 *   gbb_dequant: the affine dequantization of the MixLLM page, section 2.1:
 *   w32 device fp32 [N][K] = (q - z) * s (exact), and/or w16
 *   device fp16 [N][K] = its round-to-nearest-even (either may be NULL). */
gbb_status gbb_unpack_codes(const void* image, int N, int K, uint8_t* q, void* stream);
gbb_status gbb_dequant(const void* image, int N, int K, float* w32, uint16_t* w16,
                       void* stream);

/* ------------------------------------------------------------------------ */
/* 64x64 blocks (the other GPU block size of the ScaleBITS explainer page,  */
/* section 4.2): 64 output rows x 64 input columns per block, one bitwidth  */
/* per block, scale/zero per (row, 64-column group).  The image is version  */
/* 2 of the block image: 512 * b bytes of codes per block.  Each call below */
/* is its 64x128 counterpart's with K a multiple of 64 and bits [N/64][K/64].*/
/* ------------------------------------------------------------------------ */
size_t gbb_packed_bytes_64x64(const uint8_t* bits, int N, int K);
gbb_status gbb_pack_blocks_64x64(const uint16_t* W, int N, int K, const uint8_t* bits,
                                 uint16_t* scale, uint16_t* zero, unsigned flags,
                                 void* image, size_t image_cap);
/* y = x . dequant(W)^T over a version-2 image, with the arguments, layout,
 * workspace rules and errors of gbb_gemm_mixed_w / gbb_gemm_mixed_w_path
 * (K % 64 == 0).  M <= 32 runs the 64x64 decode kernels; larger M runs the
 * 64x64 prefill kernel (M * K < 2^31; K split into segments of at least
 * 1024 columns as for 64x128 blocks), or the decode kernels in 32-token
 * chunks under the same rule as for 64x128 blocks.  path: 0 that choice, 1 the decode
 * kernel (M <= 32), 2 the prefill kernel. */
size_t gbb_gemm_mixed_w_64x64_workspace(int N, int K, int M);
gbb_status gbb_gemm_mixed_w_64x64(const void* image, int N, int K, const uint16_t* x,
                                  uint16_t* y, int M, void* workspace, size_t ws_bytes,
                                  void* stream);
size_t gbb_gemm_mixed_w_64x64_path_workspace(int N, int K, int M, int path);
gbb_status gbb_gemm_mixed_w_64x64_path(const void* image, int N, int K, const uint16_t* x,
                                       uint16_t* y, int M, void* workspace, size_t ws_bytes,
                                       int path, void* stream);
gbb_status gbb_unpack_codes_64x64(const void* image, int N, int K, uint8_t* q, void* stream);
gbb_status gbb_dequant_64x64(const void* image, int N, int K, float* w32, uint16_t* w16,
                             void* stream);

/* ======================================================================== */
/* Output-feature mixed format, W8 (symmetric) / W4 (asymmetric) x A8       */
/* ======================================================================== */

/* Byte size of the W4/W8 image for N x K with n8 8-bit rows (0 on error):
 * the output-feature mixed format of the MixLLM page, sections 3.1.1 and
 * 3.1.2, pre-packed as in section 3.3. */
size_t gbb_w48_packed_bytes(int N, int K, int n8);

/* Quantize and pack (host, synchronous, deterministic).
 *   W      host fp16 [N][K], K % 128 == 0.
 *   rows8  host int32 [n8], strictly ascending output rows that get 8-bit
 *          symmetric codes (s = fp16(max|w| / 127), q = clamp(rint(w / s),
 *          -127, 127)); every other row gets 4-bit asymmetric codes as in
 *          gbb_pack_blocks (MixLLM page, sections 3.1.1 and 3.1.2).
 *   scale  host fp16 [N][K/128] output in original row order (may be NULL).
 *   zero   host uint8 [N][K/128] output, 0 for 8-bit rows (may be NULL).
 *   image  host output of gbb_w48_packed_bytes(N, K, n8) bytes. */
gbb_status gbb_pack_w48(const uint16_t* W, int N, int K, const int32_t* rows8, int n8,
                        uint16_t* scale, uint8_t* zero, void* image, size_t image_cap);

/* 8-bit symmetric activation quantization (MixLLM page, section 3.1.2):
 * per token (ga == K) or per group of 128 columns (ga == 128).  Decisions in
 * fp32: s = fp16(max|x| / 127) (1 if the group is all zero),
 * xq = clamp(rint(x / s), -127, 127).
 *   x  device fp16 [M][K];  xq device int8 [M][K];  xs device fp16 [M][K/ga]. */
gbb_status gbb_quant_act_i8(const uint16_t* x, int M, int K, int ga, int8_t* xq,
                            uint16_t* xs, void* stream);

/* y = dequant(xq) . dequant(W)^T by two-step dequantization (MixLLM page,
 * section 3.3): per 128-group an exact int32 product xq . (q - z) on the int8
 * matrix cores, then scaled by s_a * s_w and accumulated in fp32; each output
 * is written straight to its original row (fused scatter).
 *   image  device copy of gbb_pack_w48's output.
 *   xq, xs as produced by gbb_quant_act_i8 with the same ga (K or 128).
 *   y      device fp16 [M][N]. */
gbb_status gbb_gemm_w48a8(const void* image, int N, int K, int n8, const int8_t* xq,
                          const uint16_t* xs, int ga, uint16_t* y, int M, void* stream);

/* Workspace bytes for gbb_gemm_w48a8_split (0 when the call does not split
 * K, or on invalid arguments): the fp32 partial sums of the K split,
 * segments x M x padded rows x 4 bytes (M at most 64, the tokens of one pass,
 * on the streaming kernel; padded rows: each of the two row sets rounded up
 * to a multiple of 16). */
size_t gbb_gemm_w48a8_workspace(int N, int K, int n8, int M, int ga);

/* gbb_gemm_w48a8 with a caller workspace, for batches on matrices with few
 * output rows per compute unit (MixLLM page, section 3.3: the same
 * two-step product over a K range cut into segments).  The streaming kernel
 * (M <= 64 per pass; per-token activation scales, or per-group ones over an
 * even number of groups with xs 4-byte aligned) splits K where its 64-row
 * blocks, an 8-bit one counted twice, number at most 3/4 of the compute
 * units; it then streams 128-row blocks, and each one's 128-column groups
 * are cut into up to 16 segments of at least 8 groups, an 8-bit row block
 * into twice as many as a 4-bit one, so that every workgroup streams about
 * the same bytes.  The tile
 * kernel (larger M) splits K where its token tiles x row blocks fill at most
 * half of its resident workgroups, a 4-bit row block (twice the rows)
 * counted twice and cut into twice the segments.  Each segment writes its
 * fp32 sum of s_w-scaled group products (with per-group activation scales,
 * of s_a s_w-scaled ones) for every output to the workspace; a second
 * launch adds the segments in order, multiplies by the per-token s_a,
 * rounds to fp16, writes each output to its original row and clears the
 * workspace.  With a workspace smaller than gbb_gemm_w48a8_workspace(N, K,
 * n8, M, ga) (or NULL) the call takes as many segments as fit, down to none
 * (then it equals gbb_gemm_w48a8).  The segment counts fix the order of the
 * fp32 sums: for one ws_bytes the result is the same on every call.
 *   workspace/ws_bytes  device memory, 16-byte aligned, zero-filled before
 *          its first use (every call leaves it zero); calls that may overlap
 *          need separate workspaces.
 * Errors: those of gbb_gemm_w48a8; GBB_E_ALIGN for a misaligned workspace. */
gbb_status gbb_gemm_w48a8_split(const void* image, int N, int K, int n8, const int8_t* xq,
                                const uint16_t* xs, int ga, uint16_t* y, int M, void* workspace,
                                size_t ws_bytes, void* stream);

/* Debug export of the first step of the two-step dequantization (MixLLM
 * page, section 3.3: per group an exact integer product of the int8
 * activations and the int8 weight codes (q - z), before any scale):
 * acc[m][n][g] = sum over group g of xq[m][k] * (q[n][k] - z[n][g]) for every
 * original row n (device int32 [M][N][K/128]), for bit-exact tests.  The call
 * runs the kernel gbb_gemm_w48a8 runs for the same M and ga (K or 128), with
 * that kernel's scaling step replaced by a store of the group sums, so the
 * integers checked are those the product path forms (where the product
 * kernel starts a group's sums from the constant 0x4B400000 so that the
 * result reads as a float, its integers are these plus that constant); the
 * streaming kernel runs with the K segments that gbb_gemm_w48a8_split takes
 * with a full workspace.  Errors as gbb_gemm_w48a8. */
gbb_status gbb_w48_group_acc(const void* image, int N, int K, int n8, const int8_t* xq, int ga,
                             int32_t* acc, int M, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GBB_H */
