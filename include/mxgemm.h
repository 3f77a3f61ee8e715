/*
 * mxgemm.h - C ABI of the MXFP6 block-scaled GEMM library for AMD Instinct
 * MI355X (gfx950, CDNA4).
 *
 * What it computes.  The Hedra post "Optimizing Krea 3 on AMD Instinct MI355X
 * with AI researchers" moves the diffusion transformer's MLPs to MXFP6
 * (section "Quality set the precision limit": 6-bit floating-point elements
 * that share one scale per block) and replaces the library GEMM with a custom
 * MXFP6 GEMM (section "We built a faster MXFP6 kernel": packed 6-bit storage,
 * no re-reads by neighbouring workgroups, Figure 1 timings).  In its section
 * "Fusion cut intermediate memory traffic" the MLP's second GEMM takes the
 * first one's output already in MXFP6, with no bf16 copy written and
 * re-quantized in between.  The pages fix no element variant, block
 * size or rounding; this library follows the OCP Microscaling (MX) v1.0
 * definition:
 *
 *   - a block is 32 consecutive elements of one row along the reduction
 *     dimension K (for a quantized GEMM output: along N);
 *   - each block has one E8M0 scale byte u, value 2^(u-127); u = 0xFF is NaN;
 *   - u = clamp(floor(log2(max |v|)) - emax_elem, -127, 127) + 127, with
 *     emax_elem = 2 for E2M3 and 4 for E3M2; an all-zero block gets u = 0;
 *   - each element is v / 2^(u-127) rounded to the nearest FP6 value, ties to
 *     even, magnitudes above the largest (7.5 for E2M3, 28 for E3M2)
 *     saturate; the sign bit is the source's sign bit (so -0.0 -> 0b100000);
 *   - a block containing a NaN or an infinity gets u = 0xFF and codes 0.
 *
 * The same section weighs MXFP4 (which the chip runs at the MXFP6 rate) and
 * FP8 against MXFP6.  The library also takes the other element types of the
 * gfx950 scaled matrix instruction, with the same block, scale and rounding
 * rule: E2M1 (FP4: emax_elem 2, max 6), E4M3 (FP8: emax_elem 8, max 448) and
 * E5M2 (FP8: emax_elem 15, max 57344).  Their special codes (E4M3's NaN,
 * E5M2's infinities and NaNs) are never produced: larger finite magnitudes
 * saturate to the maximum, and non-finite blocks get u = 0xFF and codes 0.
 *
 * The skinny split-K GEMM follows the split-K technique of the page "Creating
 * Custom Kernels for the AMD MI300" (section "Skinny GEMM Kernel"): K is cut
 * into contiguous chunks computed concurrently and their fp32 partial sums are
 * reduced in a fixed order.
 *
 * Packing.  With b-bit codes (b = 6, 4 or 8), element i of a row occupies
 * bits [b*i, b*i+b) of the row read as a little-endian bit string, so a
 * 32-element block is 4b bytes (24, 16 or 32).  For b = 6 four codes c0..c3
 * form the 24-bit word c0 | c1<<6 | c2<<12 | c3<<18; for b = 4 byte i holds
 * element 2i in its low nibble and element 2i+1 in its high nibble.  Code
 * bits: sign (the top bit), then the exponent field, then the mantissa field.  Weights use the
 * PyTorch Linear layout [N, K]; the GEMM computes C[M, N] = A[M, K] * W[N, K]^T
 * with exact block-scaled products and fp32 accumulation.  All buffers are
 * owned by the caller and live in device memory.  Two storage layouts:
 *
 * MX_LAYOUT_ROWS (interchange):
 *   codes   [rows, bK/8] bytes, row-major (row r is the packed row above);
 *   scales  [rows, K/32] bytes, row-major.
 *
 * MX_LAYOUT_TILED (the operand layout of both GEMMs and of the MX output): the
 * matrix is cut into stages of 128 K-elements (S = ceil(K/128)) and groups of
 * 32 rows (G = ceil(rows/32)).  Each (stage s, group g) pair owns, for the
 * 6-bit types,
 *   codes   3072 bytes at offset (s*G + g) * 3072.  For each row j = 0..31 of
 *           the group, the row's 96-byte packed slice of K-elements
 *           [128s, 128s+128) is four 24-byte blocks q = 0..3.  Half h = 0, 1
 *           of the chunk (bytes [1536h, 1536h+1536)) holds blocks 2h and 2h+1
 *           of all 32 rows in four planes:
 *             +0     plane A: bytes 0..15 of block 2h,   row j at j*16;
 *             +512   plane L: bytes 16..23 of block 2h,  row j at j*8;
 *             +768   plane H: bytes 0..7 of block 2h+1,  row j at j*8;
 *             +1024  plane B: bytes 8..23 of block 2h+1, row j at j*16;
 *           so each block of a row is one 16-byte and one 8-byte run;
 *   scales  128 bytes at offset (s*G + g) * 128: byte j*4 + q is the scale of
 *           block 4s+q of row 32g+j.
 *   For the 8-bit types a chunk is 4096 bytes at offset (s*G + g) * 4096;
 *   half h (bytes [2048h, 2048h+2048)) holds bytes 16h..16h+15 of every
 *   block of the 32 rows in four planes of 16 bytes per row (row j at j*16):
 *             +0     block 0,   +512   block 2,
 *             +1024  block 1,   +1536  block 3
 *   (the instruction takes each 8-bit block from both lane halves).
 *   For E2M1 a chunk is 2048 bytes at offset (s*G + g) * 2048; half h
 *   (bytes [1024h, 1024h+1024)) holds block 2h at +0 and block 2h+1 at +512,
 *   16 bytes per row (row j at j*16).  The scales are the same for all types.
 *   Rows >= rows and blocks >= K/32 are padding: codes 0, scale byte 127.
 *   Total: codes S*G*512b bytes (3072 for the 6-bit types), scales S*G*128
 *   bytes (mx_packed_bytes).  Each stage of 256 rows is one contiguous run
 *   (24 KB for the 6-bit types), which the GEMM copies straight into its LDS
 *   ring.
 *
 * Conventions:
 *   - every call is asynchronous on the given HIP stream; the library never
 *     allocates, frees or synchronizes device memory, and keeps no mutable
 *     global state, so calls on different streams may run concurrently as
 *     long as their buffers do not overlap.  The one exception is
 *     mx_gemm_splitk_noalloc, whose calls on one GPU share a static device
 *     scratch array (see there);
 *   - within one call, outputs (out, out_scales, codes, scales, the
 *     workspace) must not overlap each other or any input: inputs are read
 *     while outputs are written, and overlapping buffers are not detected;
 *   - argument errors are detected on the host before anything is launched
 *     and return a negative status; nothing is written in that case;
 *   - MX_ERR_HIP reports a failed launch (hipGetLastError); a fault inside a
 *     kernel surfaces at the caller's next synchronization instead;
 *   - device pointers must be 16-byte aligned unless stated otherwise;
 *   - size limits: every dimension, leading dimensions included, is at most
 *     2^30 (else MX_ERR_SHAPE).
 *     Beyond that a request returns MX_ERR_UNSUPPORTED, before anything is
 *     launched, when a tiled MX matrix would hold 2^40 code bytes or more,
 *     when one 128-element stage of a GEMM operand (all its rows) would reach
 *     4 GiB, or when a kernel would need 2^32 lanes or more (a dispatch holds
 *     its grid size in 32 bits).  Inside those limits every byte offset is
 *     computed in 64 bits, so buffers may be far larger than 4 GiB;
 *   - the header is plain C99 as well as C++: a C program compiles it with
 *     -D__HIP_PLATFORM_AMD__ -I/opt/rocm/include (what hipcc passes, for
 *     hipStream_t) and links -lmxgemm; tests/abi_from_c.c does exactly that;
 *   - launch log: with the environment variable MXGEMM_LOG=1 (read once, at
 *     the first call), every call of mx_quantize, mx_rmsnorm_quantize,
 *     mx_gemm, mx_gemm_with_config, mx_gemm_splitk and
 *     mx_gemm_splitk_noalloc writes one line to stderr: the call, its sizes,
 *     formats and options (for mx_gemm the launch configuration and whether
 *     the shape rule chose it) and the status returned.  Off otherwise.
 */
#ifndef MXGEMM_H
#define MXGEMM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MX_OK 0
#define MX_ERR_NULL (-1)        /* a required pointer is NULL                        */
#define MX_ERR_SHAPE (-2)       /* negative size, K % 32 != 0, ld too small, ...     */
#define MX_ERR_FORMAT (-3)      /* unknown element format / source / output kind     */
#define MX_ERR_ALIGN (-4)       /* a pointer or leading dimension breaks alignment   */
#define MX_ERR_WORKSPACE (-5)   /* workspace NULL or smaller than required           */
#define MX_ERR_UNSUPPORTED (-6) /* valid request with no kernel variant              */
#define MX_ERR_HIP (-7)         /* a kernel launch failed                            */
#define MX_ERR_SCRATCH (-8)     /* larger than mx_gemm_splitk_noalloc's static scratch */

/* Element formats.  The values equal the format codes of the gfx950 scaled
 * f8f6f4 MFMA instructions. */
#define MX_FMT_E4M3 0 /* FP8 */
#define MX_FMT_E5M2 1 /* FP8 */
#define MX_FMT_E2M3 2 /* FP6 */
#define MX_FMT_E3M2 3 /* FP6 */
#define MX_FMT_E2M1 4 /* FP4 */

/* Storage layouts of packed MX matrices. */
#define MX_LAYOUT_ROWS 0
#define MX_LAYOUT_TILED 1

/* Source types for quantization. */
#define MX_SRC_BF16 0
#define MX_SRC_F32 1

/* GEMM output kinds. */
#define MX_OUT_F32 0  /* fp32 C                                              */
#define MX_OUT_BF16 1 /* bf16 C, round-to-nearest-even                        */
#define MX_OUT_MX 2   /* MX codes + scales of the epilogue's result, along N  */

/* GEMM epilogues. */
#define MX_EPI_NONE 0
#define MX_EPI_GELU_TANH 1 /* 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) */
/* SwiGLU over stacked gate/up weights (the MLP activation of the Hedra post,
 * section "Fusion cut intermediate memory traffic"; silu(x) = x / (1 + e^-x)):
 * W holds n = 2h rows in runs of 128, the first 64 rows of each run are the
 * gate rows of 64 consecutive features and the next 64 the up rows of the
 * same features, i.e. feature f's gate row is 128 * (f / 64) + f % 64 and its
 * up row is 64 rows later.  The output has h = n / 2 features:
 * out[:, f] = silu(C[:, gate row f]) * C[:, up row f]. */
#define MX_EPI_SWIGLU 2

/*
 * mx_quantize - MX-quantize a [rows, k] matrix along its rows.
 *
 * This is the activation quantizer of the Hedra post's section "Fusion cut
 * intermediate memory traffic" (an activation is quantized once and every
 * GEMM that consumes it reads the packed result), with the block, scale and
 * rounding rule of the header comment.  It also quantizes weights once,
 * ahead of the GEMMs that read them.
 *
 *   src       device pointer to bf16 (src_type MX_SRC_BF16) or fp32
 *             (MX_SRC_F32) values, row r starting at src + r * ld_src
 *             elements; 16-byte aligned, ld_src * element size a multiple of 16.
 *   rows, k   rows >= 0, k >= 0, k % 32 == 0.  rows == 0 or k == 0 is a
 *             no-op that returns MX_OK.
 *   fmt       any MX_FMT_* element format.
 *   layout    MX_LAYOUT_ROWS or MX_LAYOUT_TILED (padding included).
 *   codes     device output of mx_packed_bytes(rows, k, fmt, layout, 0)
 *             bytes, 16-byte aligned.
 *   scales    device output of mx_packed_bytes(rows, k, fmt, layout, 1)
 *             bytes, 4-byte aligned.
 * The result is exactly the rule in the header comment (bit-exact).
 */
int mx_quantize(const void* src, int32_t src_type, int64_t rows, int64_t k, int64_t ld_src, int32_t fmt,
                int32_t layout, void* codes, uint8_t* scales, hipStream_t stream);

/*
 * mx_rmsnorm_quantize - the quantize-once producer of a GEMM's activations:
 * RMSNorm, the adaptive-norm modulation, and MX quantization in one pass
 * (the Hedra post, section "Fusion cut intermediate memory traffic": the
 * modulation and RMSNorm producers are fused and the activations are
 * quantized once).  For each row r of x:
 *
 *   inv    = 1 / sqrt(mean_k x[r,k]^2 + eps)
 *   y[r,k] = x[r,k] * inv * gamma[k] * (1 + scale[c,k]) + shift[c,k],
 *            c = r / rows_per_cond,
 *
 * evaluated in fp32, then y is MX-quantized along the row exactly as
 * mx_quantize quantizes an fp32 source, into MX_LAYOUT_TILED.
 *
 *   x         device bf16 (src_type MX_SRC_BF16) or fp32 [rows, d], row r at
 *             x + r * ld_x elements; 16-byte aligned, ld_x * element size a
 *             multiple of 16.
 *   rows, d   rows >= 0, d >= 0, d % 32 == 0; rows == 0 or d == 0 is a no-op.
 *   gamma     device fp32 [d] gain, or NULL for ones.
 *   shift, scale  device fp32 [ceil(rows / rows_per_cond), d] modulation
 *             vectors, either may be NULL (zeros).  When either is given,
 *             rows_per_cond must be a positive multiple of 32 (every 32-row
 *             group of the output shares one conditioning row); otherwise it
 *             is ignored.
 *   eps       >= 0, finite.
 *   fmt       MX_FMT_E2M3 or MX_FMT_E3M2 (other formats: MX_ERR_UNSUPPORTED).
 *   codes, scales  outputs of mx_packed_bytes(rows, d, fmt, MX_LAYOUT_TILED,
 *             0 / 1) bytes (16- and 4-byte aligned), padding included.
 * The result follows the fp32 evaluation above; it is not bit-identical to a
 * float64 evaluation where y lies at a rounding boundary of its code.
 */
int mx_rmsnorm_quantize(const void* x, int32_t src_type, int64_t rows, int64_t d, int64_t ld_x, const float* gamma,
                        const float* shift, const float* scale, int64_t rows_per_cond, float eps, int32_t fmt,
                        void* codes, uint8_t* scales, hipStream_t stream);

/*
 * mx_packed_bytes - size in bytes of the codes (which == 0) or scales
 * (which == 1) buffer of a [rows, k] MX matrix of element format fmt in the
 * given layout; 0 for invalid arguments.
 */
size_t mx_packed_bytes(int64_t rows, int64_t k, int32_t fmt, int32_t layout, int32_t which);

/*
 * mx_gemm - C = A * W^T on MX operands, fp32 accumulation, optional epilogue.
 *
 * Activations: exactly one of
 *   a_src  (bf16 or fp32 [m, k] at a_src + r * lda elements, quantized to
 *          a_fmt inside the call into the workspace before the GEMM), or
 *   a_codes / a_scales (already quantized, format a_fmt, MX_LAYOUT_TILED).
 * Weights: w_codes / w_scales of the [n, k] weights in MX_LAYOUT_TILED,
 *   format w_fmt.
 * Alignment: a_src and code pointers 16 bytes, scale pointers 4 bytes, the
 *   workspace 256 bytes, f32/bf16 outputs their element size (16 bytes and
 *   ldo * element size % 16 == 0 enable vector stores), MX outputs 4 bytes.
 * Formats (weights x activations): E2M3 x E2M3, E2M3 x E3M2 and E3M2 x
 *   E2M3 with every epilogue and output; E2M1 x E2M1, and E4M3 / E5M2 x
 *   E4M3 / E5M2, with MX_EPI_NONE and MX_OUT_F32 / MX_OUT_BF16.  Other pairs
 *   (E3M2 x E3M2, where the scaled MFMA does not keep fp32 accuracy, and
 *   pairs of different element widths) return MX_ERR_UNSUPPORTED.
 * m, n, k: >= 0, k % 32 == 0.  m == 0 or n == 0 is a no-op; k == 0 writes
 *   C = 0 (epilogue applied).
 * epilogue: MX_EPI_NONE, MX_EPI_GELU_TANH or MX_EPI_SWIGLU, applied to the
 *   fp32 accumulator.  MX_EPI_SWIGLU needs n % 128 == 0 and produces
 *   n_out = n / 2 output features; the other epilogues keep n_out = n.
 * out_kind:
 *   MX_OUT_F32 / MX_OUT_BF16: out is [m, ldo] elements (ldo >= n_out), the
 *     result is written to its first n_out columns; out_scales, out_fmt are
 *     ignored.
 *   MX_OUT_MX: the epilogue result is MX-quantized along N in blocks of 32
 *     (n_out % 32 == 0) into out / out_scales as an [m, n_out] matrix in
 *     MX_LAYOUT_TILED (padding written too), element format out_fmt
 *     (MX_FMT_E2M3 or MX_FMT_E3M2); ldo is ignored.  This output is directly the
 *     a_codes / a_scales of a following GEMM, which reads it with no bf16
 *     round trip.
 * workspace: device memory of at least mx_gemm_workspace_size(m, n, k, a_src
 *   != NULL, 0) bytes (may be NULL when that size is 0).  That size holds the
 *   quantized activations in any element format.
 */
int mx_gemm(const void* a_src, int32_t a_src_type, int64_t lda, const void* a_codes, const uint8_t* a_scales,
            int32_t a_fmt, const void* w_codes, const uint8_t* w_scales, int32_t w_fmt, int64_t m, int64_t n,
            int64_t k, int32_t epilogue, int32_t out_kind, void* out, int64_t ldo, uint8_t* out_scales,
            int32_t out_fmt, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Launch configuration of mx_gemm: the tile width, the waves per workgroup
 * and the order in which the tiles are handed to workgroups.  It changes the
 * speed (which operand stages the workgroups in flight share in each XCD's
 * L2, how many workgroups share a CU), never the result: every configuration
 * computes each output with the same arithmetic (the same MFMA sequence over
 * K per output).  The Hedra post (section "We tuned before writing custom
 * kernels") keeps per-shape choices found by timing candidates on real data;
 * a table of such choices (microscaled_precision_gemm_amd/tuning.py, with the
 * one tuned on MI355X in tuned_gfx950.json) passes them here.
 */
typedef struct {
  int32_t group_m;   /* m-tiles per group of the tile walk, 1 .. 16 (default 4)             */
  int32_t xcd_remap; /* 1: each XCD walks a contiguous range of the grouped order (default);
                        0: tiles in plain grouped order, dealt round-robin to the XCDs        */
  int32_t tile_n;    /* weight rows per tile (output features; with MX_EPI_SWIGLU stacked
                        gate/up rows, i.e. twice the output features): 256 (default; 4 waves
                        of 128 x 128, one workgroup per CU) or 128 (4 waves of 128 x 64 and a
                        two-slot LDS ring, two workgroups per CU, so one's prologue, waits and
                        epilogue overlap the other's matrix work; the 6-bit format pairs
                        only, else MX_ERR_UNSUPPORTED)                                      */
  int32_t waves;     /* waves per workgroup: 4 (default) or, with tile_n = 256, 8 (2 x 4 waves
                        of 128 x 64, two per SIMD, sharing the tile's operand ring; any format
                        pair and epilogue; with tile_n = 128, MX_ERR_UNSUPPORTED)             */
} mx_gemm_config;

/* mx_gemm_default_config - fill *config with the generic configuration
 * (group_m 4, xcd_remap 1, tile_n 256, 4 waves): the one every format pair and
 * epilogue takes. */
void mx_gemm_default_config(mx_gemm_config* config);

/*
 * mx_gemm_select_config - fill *config with the configuration mx_gemm uses
 * for a call of this shape when it is given none (a shape rule, so that a
 * shape missing from a tuning table does not fall back to the generic
 * configuration; the Hedra post, section "We tuned before writing custom
 * kernels", found library GEMMs doing exactly that).  The rule, from timings
 * of every candidate on the workload shapes on MI355X:
 *   - FP8 operands: the generic configuration;
 *   - otherwise (4- and 6-bit operands): 8 waves on 256-feature tiles, with
 *     group_m 8 for MX_OUT_MX after MX_EPI_NONE or MX_EPI_GELU_TANH and
 *     group_m 4 otherwise.
 * Arguments as mx_gemm's; nothing is validated (an invalid call still fails
 * in mx_gemm).
 */
void mx_gemm_select_config(int64_t m, int64_t n, int64_t k, int32_t a_fmt, int32_t w_fmt, int32_t epilogue,
                           int32_t out_kind, mx_gemm_config* config);

/*
 * mx_gemm_with_config - mx_gemm with an explicit launch configuration
 * (NULL = mx_gemm_select_config's choice, which is what mx_gemm uses).  Same
 * arguments, results and errors as mx_gemm, plus MX_ERR_FORMAT for a
 * configuration outside the ranges above.
 */
int mx_gemm_with_config(const void* a_src, int32_t a_src_type, int64_t lda, const void* a_codes,
                        const uint8_t* a_scales, int32_t a_fmt, const void* w_codes, const uint8_t* w_scales,
                        int32_t w_fmt, int64_t m, int64_t n, int64_t k, int32_t epilogue, int32_t out_kind, void* out,
                        int64_t ldo, uint8_t* out_scales, int32_t out_fmt, void* workspace, size_t workspace_bytes,
                        const mx_gemm_config* config, hipStream_t stream);

/*
 * mx_gemm_splitk - the same product for skinny m (0 <= m <= 16), split along
 * K into `splits` contiguous chunks whose fp32 partial sums are added in the
 * fixed order 0, 1, ..., splits-1 (deterministic) before the output rounding.
 * This is the split-K scheme of "Creating Custom Kernels for the AMD MI300",
 * section "Skinny GEMM Kernel": with few rows there are too few output tiles
 * to occupy every compute unit, so the reduction dimension is divided among
 * workgroups instead.
 *
 * Arguments as mx_gemm (operands in MX_LAYOUT_TILED), with:
 *   splits    1 .. 16 and k % (128 * splits) == 0, i.e. each chunk is whole
 *             128-element stages (else MX_ERR_UNSUPPORTED); m <= 16 (else
 *             MX_ERR_SHAPE).
 *   formats   the 6-bit pairs of mx_gemm only (else MX_ERR_UNSUPPORTED).
 *   epilogue  MX_EPI_NONE only; out_kind MX_OUT_F32 or MX_OUT_BF16.
 *   workspace at least mx_gemm_workspace_size(m, n, k, a_src != NULL, splits)
 *             bytes, used for the activations quantized inside the call (the
 *             partial sums stay on chip); may be NULL when that size is 0.
 */
int mx_gemm_splitk(const void* a_src, int32_t a_src_type, int64_t lda, const void* a_codes,
                   const uint8_t* a_scales, int32_t a_fmt, const void* w_codes, const uint8_t* w_scales,
                   int32_t w_fmt, int64_t m, int64_t n, int64_t k, int32_t splits, int32_t out_kind, void* out,
                   int64_t ldo, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mx_gemm_splitk_noalloc - mx_gemm_splitk for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  It takes no workspace and allocates
 * nothing (no hipMalloc / hipFree, no allocating library routine).  The
 * activations it quantizes inside the call go to a file-scope device array
 * of the library (1.5625 MiB: one 32-row group of k <= MX_NOALLOC_MAX_K
 * 6-bit codes and their scales), which each GPU the library runs on holds
 * until the process ends; its address is looked up once per device, on the
 * first call with that device current.  The array used is the one of the
 * device current in the calling thread, so `stream` must belong to that
 * device (unlike the other calls, which follow the stream).  The caller still
 * owns a_src / the quantized operands, the weights and out.
 *
 * Arguments, results and errors as mx_gemm_splitk without the workspace
 * (the results are bit-identical to it), plus MX_ERR_SCRATCH when
 * k > MX_NOALLOC_MAX_K.  Every call on one GPU shares that GPU's array and
 * leaves its last contents there: calls that overlap in time on one GPU
 * (different streams, or host threads without ordering) race on it and must
 * be serialized by the caller; calls on one stream are ordered.
 */
#define MX_NOALLOC_MAX_K 65536
int mx_gemm_splitk_noalloc(const void* a_src, int32_t a_src_type, int64_t lda, const void* a_codes,
                           const uint8_t* a_scales, int32_t a_fmt, const void* w_codes, const uint8_t* w_scales,
                           int32_t w_fmt, int64_t m, int64_t n, int64_t k, int32_t splits, int32_t out_kind,
                           void* out, int64_t ldo, hipStream_t stream);

/*
 * mx_gemm_workspace_size - bytes of workspace needed by mx_gemm (splits == 0)
 * or mx_gemm_splitk (splits >= 1) for these sizes; a_is_src != 0 when the
 * activations are passed unquantized.  Returns 0 for invalid sizes.
 */
size_t mx_gemm_workspace_size(int64_t m, int64_t n, int64_t k, int32_t a_is_src, int32_t splits);

/* mx_status_string - static, human-readable text for a status code. */
const char* mx_status_string(int status);

/* mx_version - library version as major * 10000 + minor * 100 + patch. */
int mx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXGEMM_H */
