/*
 * convrot.h -- C-ABI of libconvrot, the ConvRot quantized linear layer for AMD MI355X (gfx950).
 *
 * What the layer computes (sources are the pages this library follows):
 *   ConvRot rotates a weight by a Hadamard transform over fixed groups of input channels before
 *   quantizing it, which spreads outlier energy so INT8 can hold it, and the GEMM then runs on
 *   INT8 tensor cores ("minimax-h3-nvfp4-convrot核心原理", section 四 "核心原理 3：INT8 ConvRot").
 *   The group is 256 channels (same section, detail 3; converter flag --convrot-group-size 256 in
 *   "Qwen3-VL-32B-...-INT8-ConvRot部署优化", section 量化转换过程), INT8 weights carry one FP32
 *   scale per output row (--scaling_mode row there; "INT8 row-scale" in section 四), and the
 *   W4A4 variant rotates activations and weights alike and quantizes both to 4 bits with
 *   round-to-nearest (nvfp4-convrot page, section 五 "INT4 W4A4 ConvRot").
 *
 *   R       = blockdiag(H_g / sqrt(g), ...) along K, H_g the Sylvester Hadamard matrix
 *             (H[i][j] = (-1)^popcount(i & j)), g a power of two, groups contiguous along K.
 *   INT8:   s = max|v R| / 127 per row (fp32),  q = rint(v R / s) in [-127, 127]
 *   INT4:   s = max|v R over a g-group| / 7 per (row, group) (fp16), c = rint(v R / s) in [-7, 7]
 *   linear: y[m,n] = bf16( sum_k xq[m,k] wq[n,k] * sx[m] * sw[n] + bias[n] )          (INT8)
 *           y[m,n] = bf16( sum_j (sum_{k in group j} cx cw) * sx[m,j] * sw[n,j] + bias[n] ) (W4A4)
 *   Because R is orthogonal, (x R)(w R)^T = x w^T, so the integer product of rotated codes
 *   approximates x w^T.  Rounding is to nearest even; a zero row/group has scale 0, codes 0.
 *
 * Conventions (all entry points):
 *   - Every matrix is row-major with K contiguous.  Weights are [N, K] = [out, in].
 *   - Pointers named x/w/xq/wq/y/scale/bias/workspace are DEVICE pointers owned by the caller;
 *     the library allocates and frees nothing.  Matrix pointers must be 16-byte aligned, fp32
 *     scale/bias pointers 4-byte aligned, fp16 scale pointers 2-byte aligned.
 *   - Work is enqueued on `stream` (NULL = the default stream) and returns without waiting.
 *     A fault inside a kernel surfaces at the caller's next synchronisation.
 *   - Preconditions are checked on the host before anything is launched: a violated one returns
 *     a non-zero status and enqueues nothing.  convrot_last_error() then describes it.
 *   - Shapes: 0 <= M, N < 2^31; 64 <= K <= 131072 and K % 64 == 0; 1 <= group <= 256 a power of
 *     two dividing K.  M == 0 or N == 0 is a no-op that returns CONVROT_OK.
 *   - Inputs must be finite.  The library is stateless and thread-safe, except that one
 *     workspace buffer must not be used by two calls that may run concurrently.
 */
#ifndef CONVROT_H
#define CONVROT_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum convrot_status {
    CONVROT_OK = 0,
    CONVROT_ERR_NULL = 1,      /* a required pointer is NULL                                   */
    CONVROT_ERR_SHAPE = 2,     /* M, N or K out of range, K % 64 != 0, or K % group != 0         */
    CONVROT_ERR_GROUP = 3,     /* group not a power of two in [1, 256] (INT4: 256 or 128)        */
    CONVROT_ERR_ALIGN = 4,     /* a pointer violates the alignment rules above                   */
    CONVROT_ERR_DTYPE = 5,     /* unknown dtype code                                             */
    CONVROT_ERR_BITS = 6,      /* bits is not 8 or 4                                             */
    CONVROT_ERR_WORKSPACE = 7, /* workspace NULL, misaligned or smaller than the call requires  */
    CONVROT_ERR_HIP = 8,       /* a HIP runtime call or kernel launch failed                     */
    CONVROT_ERR_DEVICE = 9     /* the current device is not gfx950                               */
} convrot_status;

enum { CONVROT_DTYPE_F32 = 0, CONVROT_DTYPE_BF16 = 1 };

#define CONVROT_MAX_K 131072
/* The tiled GEMMs (the W8A8 linear at M > 16 and every W4A4 call) need N < CONVROT_GEMM_MAX_N:
 * their epilogue addresses a 32-row block of the output with a 32-bit byte offset.  The decode
 * GEMVs (M <= 16) take any N < 2^31.  A larger N returns CONVROT_ERR_SHAPE. */
#define CONVROT_GEMM_MAX_N 16777216

/*
 * Offline weight preparation: rotate each weight row by R and quantize it
 * ("ConvRot pre-rotates the weight in fixed groups before quantization", nvfp4-convrot page,
 * section 四; quantize from the original BF16/FP32 weight, same section, detail 1).
 *   w        [N, K] fp32 or bf16 (w_dtype)
 *   bits 8:  wq int8 [N, K];        w_scale fp32 [N]
 *   bits 4:  wq uint8 [N, K/2] (two codes per byte, even k in the low nibble);
 *            w_scale fp16 [K/group, N] (group-major: scale of row n, group j at j*N + n); the
 *            scale group is the rotation group, 256 or 128 (the dynamic group of a width that 256
 *            does not divide).
 */
int convrot_prepare_weight(const void *w, int w_dtype, int64_t N, int64_t K, int group, int bits, void *wq,
                           void *w_scale, hipStream_t stream);

/*
 * Online activation quantization: rotate each token row by the same R and quantize it
 * dynamically (one scale per token for INT8, per (token, group) for INT4).  The activations get
 * the same grouped rotation as the weights (nvfp4-convrot page, section 五: the W4A4 variant
 * rotates activations and weights; on the INT8 path of section 四 the rotation cancels in the
 * product only if both operands carry it), and RTN as in section 五's --simple mode.  Same layouts as
 * convrot_prepare_weight with M rows.  Exposed so one quantized input can feed several linears
 * (for example q/k/v or gate/up projections that share an input).
 */
int convrot_quantize_act(const void *x, int x_dtype, int64_t M, int64_t K, int group, int bits, void *xq,
                         void *x_scale, hipStream_t stream);

/*
 * Workspace bytes needed by convrot_linear (bits 8) / convrot_linear_w4a4 (bits 4) for this
 * shape; 0 on invalid arguments.  The workspace must be 256-byte aligned.  It is scratch: the
 * library initialises what it needs on the stream, so any contents are fine on entry and it holds
 * nothing useful afterwards.  The bits-8 workspace holds the quantized activations (M*K bytes,
 * then 4*M, each rounded up to 256), so convrot_linear needs that much only when it quantizes x
 * itself.  For M > 16 and N % 8 == 0 it may add room for the GEMM's split-K tail (below), so
 * passing the full size is never slower.  convrot_gemm_i8_i32 needs none (it accepts and ignores
 * one); convrot_gemm_i4_i32 needs the bits-4 size.  Besides the activation
 * codes and scales, the bits-4 workspace holds both operands re-encoded as FP6 in matrix-core
 * order (1536 bytes per 32 rows x 64 channels, (ceil(M/32) + ceil(N/32)) * K/64 pieces).
 */
size_t convrot_workspace_bytes(int64_t M, int64_t N, int64_t K, int bits);

/*
 * INT8 ConvRot linear: y = bf16( (xq . wq^T) * sx[m] * sw[n] + bias[n] )   (nvfp4-convrot page,
 * section 四: INT8 row-scale weights with ConvRot metadata on the INT8 tensor-core path).
 *   x        bf16/fp32 [M, K] (x_dtype): rotated and quantized into the workspace first; or
 *   x = NULL: use the caller's xq int8 [M, K] and x_scale fp32 [M] from convrot_quantize_act.
 *   wq, w_scale from convrot_prepare_weight(bits = 8); bias fp32 [N] or NULL; y bf16 [M, N].
 * M <= 16 runs the weight-streaming GEMV, larger M the MFMA GEMM.  With x = NULL the workspace
 * may be NULL.
 * Split-K tail: the GEMM walks 256 x 256 output tiles with one persistent workgroup per CU.  When
 * the tiles leave its last round badly under-filled (few tiles: mid-size M, small N), the tail
 * tiles are computed as K-slices, their exact int32 partial sums are stored in the workspace past
 * the quantized activations, and a second kernel sums them and applies the same epilogue, so the
 * outputs are bit-identical either way.  This needs workspace_bytes >= convrot_workspace_bytes(M,
 * N, K, 8) (with x = NULL too); a smaller or NULL workspace runs without it.  The two kernels run
 * in stream order, so calls on one stream may share a workspace; calls that overlap on different
 * streams need their own.
 */
int convrot_linear(const void *x, int x_dtype, const int8_t *xq, const float *x_scale, int64_t M, int64_t N,
                   int64_t K, int group, const int8_t *wq, const float *w_scale, const float *bias, void *y,
                   void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Size of the fixed scratch array convrot_linear_noalloc uses on each GPU (32 MiB). */
#define CONVROT_NOALLOC_SCRATCH_BYTES 33554432

/*
 * convrot_linear for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments (without the workspace),
 * kernels and result bit for bit as convrot_linear.  The scratch the call needs -- the quantized
 * activations when x is given (M*K + 4*M bytes, each rounded up to 256) and, when it fits, the
 * GEMM's split-K partial sums -- lives in a fixed array of CONVROT_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends; no call allocates or frees
 * anything.  The first call on a device looks the array's address up on that device.
 * With x given, a shape whose quantized activations exceed the array returns
 * CONVROT_ERR_WORKSPACE before anything is enqueued (use convrot_linear with a workspace).
 * Every call on one GPU shares that GPU's array, and it keeps the last call's contents (each call
 * writes what it reads first, so nothing needs clearing): calls that overlap on one GPU -- on
 * different streams, or from different threads -- race on it and must be serialised by the
 * caller; calls in order on one stream are safe.
 */
int convrot_linear_noalloc(const void *x, int x_dtype, const int8_t *xq, const float *x_scale, int64_t M, int64_t N,
                           int64_t K, int group, const int8_t *wq, const float *w_scale, const float *bias, void *y,
                           hipStream_t stream);

/*
 * W4A4 ConvRot linear (nvfp4-convrot page, section 五): both operands rotated, INT4 per
 * (row, group) with fp16 scales, per-group integer dot products scaled and summed in fp32.
 *   x bf16/fp32 [M, K] rotated and quantized into the workspace (straight into the FP6
 *   matrix-core order; the same codes and scales convrot_quantize_act(bits = 4) gives, so the
 *   result is bit-identical to passing those), or x = NULL and the caller's
 *   xq uint8 [M, K/2] / x_scale fp16 [K/group, M] from convrot_quantize_act(bits = 4).
 *   The workspace (convrot_workspace_bytes(M, N, K, 4)) is required in both cases.
 *   wq uint8 [N, K/2], w_scale fp16 [K/group, N] from convrot_prepare_weight(bits = 4).
 *   group 256, or 128 for a width 256 does not divide (section 四, detail 3, dynamic group; the
 *   same group as the operands were quantized with); K % group == 0, K >= 256, N % 8 == 0.
 *   bias fp32 [N] or NULL; y bf16 [M, N].
 *   w_scale must be 8-byte aligned (the kernel reads 4 scales at a time).
 */
int convrot_linear_w4a4(const void *x, int x_dtype, const uint8_t *xq, const uint16_t *x_scale, int64_t M,
                        int64_t N, int64_t K, int group, const uint8_t *wq, const uint16_t *w_scale,
                        const float *bias, void *y, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * One-time re-encode of W4A4 weights for the matrix core (the same operation
 * convrot_linear_w4a4 performs on its weights every call, nvfp4-convrot page, section 五):
 * wq uint8 [N, K/2] from convrot_prepare_weight(bits = 4) becomes convrot_packed_bytes_w4a4(N, K)
 * bytes (16-byte aligned) of FP6 E3M2 codes in matrix-core order, 1536 bytes per 32 rows x 64
 * channels (rows past N are zero).  Every code keeps its value (-8..7 are exact E3M2 values);
 * the scales stay in w_scale, unchanged.  K % 128 == 0.
 */
int convrot_pack_weight_w4a4(const uint8_t *wq, int64_t N, int64_t K, void *w_packed, hipStream_t stream);

/* Size of the W4A4 packed weight buffer (0.75 bytes per code); 0 on invalid arguments. */
size_t convrot_packed_bytes_w4a4(int64_t N, int64_t K);

/*
 * convrot_linear_w4a4 with the weights already re-encoded by convrot_pack_weight_w4a4 (w_scale
 * as before).  Same arguments, checks and result bit for bit; the workspace needs only
 * convrot_workspace_bytes(M, 0, K, 4) bytes, since no weight codes are re-encoded per call.
 */
int convrot_linear_w4a4_packed(const void *x, int x_dtype, const uint8_t *xq, const uint16_t *x_scale, int64_t M,
                               int64_t N, int64_t K, int group, const void *w_packed, const uint16_t *w_scale,
                               const float *bias, void *y, void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Largest token count of the W4A8 decode linear. */
#define CONVROT_W4A8_MAX_M 16

/*
 * W4A8 ConvRot linear for decode-sized inputs: 4-bit weights with 8-bit activations (the
 * "MiniMax-H3-W4A8-ConvRot" tutorial page and the news page on MiniMax-H3's experimental W4A8
 * format in ComfyUI describe this format; the nvfp4-convrot page, section 七, says the W4A4
 * kernel takes an INT8-activation path on GPUs without 4-bit tensor-core MMA).  Weights keep the
 * W4A4 quantization, activations the INT8 one, both rotated by the same grouped Hadamard:
 *   y[m,n] = bf16( sx[m] * sum_j sw[j,n] * (sum_{k in group j} qx[m,k] * cw[n,k]) + bias[n] )
 *   x bf16/fp32 [M, K] rotated and quantized to INT8 into the workspace, or x = NULL and the
 *   caller's xq int8 [M, K] / x_scale fp32 [M] from convrot_quantize_act(bits = 8).
 *   w_packed: the weights in the W4A8 block layout, from convrot_pack_weight_w4a8 (group 256) or
 *   convrot_pack_weight_w4a8_group with this same group; w_packed_bytes must be exactly
 *   convrot_packed_bytes_w4a8_group(N, K, group).  The two groups' layouts differ in size for every
 *   shape, so weights packed with the other group are rejected (CONVROT_ERR_SHAPE) rather than
 *   read past their end or misread.
 *   group 256, or 128 for a width 256 does not divide (nvfp4-convrot page, section 四, detail 3,
 *   dynamic group); K % group == 0, N % 8 == 0, 0 <= M <= CONVROT_W4A8_MAX_M
 *   (CONVROT_ERR_SHAPE otherwise; larger batches belong on convrot_linear or convrot_linear_w4a4).
 *   bias fp32 [N] or NULL; y bf16 [M, N].  With x given, the workspace
 *   (convrot_workspace_bytes_w4a8 bytes, 256-byte aligned) holds the INT8 activations; with
 *   x = NULL none is needed (may be NULL).
 */
int convrot_linear_w4a8(const void *x, int x_dtype, const int8_t *xq, const float *x_scale, int64_t M, int64_t N,
                        int64_t K, int group, const void *w_packed, size_t w_packed_bytes, const float *bias, void *y,
                        void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Offline re-layout of INT4 weights for convrot_linear_w4a8: wq uint8 [N, K/2] and w_scale fp16
 * [K/256, N] from convrot_prepare_weight(bits = 4, group = 256) go into one buffer of
 * convrot_packed_bytes_w4a8(N, K) bytes (16-byte aligned), ordered the way the decode kernel
 * streams them: per 64-row tile and 256-channel block, the tile's codes (8 KiB, in MFMA operand
 * order) followed by its 64 scales; rows past N are zero.  The codes and scales are copied
 * unchanged (no requantization).  K % 256 == 0.
 */
int convrot_pack_weight_w4a8(const uint8_t *wq, const uint16_t *w_scale, int64_t N, int64_t K, void *w_packed,
                             hipStream_t stream);

/* Size of the W4A8 packed weight buffer (group 256); 0 on invalid arguments. */
size_t convrot_packed_bytes_w4a8(int64_t N, int64_t K);

/*
 * The same re-layout for either scale group: group 256 as above, or 128 (weights prepared with
 * group 128, w_scale fp16 [K/128, N]), where each 256-channel block carries two scale sets (the
 * tile's 64 scales of its lower, then of its upper 128 channels) and, when K % 256 == 128, the
 * last block's upper half is zero codes with zero scales.  K % group == 0; the buffer holds
 * convrot_packed_bytes_w4a8_group(N, K, group) bytes.  CONVROT_ERR_GROUP for another group.
 */
int convrot_pack_weight_w4a8_group(const uint8_t *wq, const uint16_t *w_scale, int64_t N, int64_t K, int group,
                                   void *w_packed, hipStream_t stream);

/* Size of the W4A8 packed weight buffer for this group; 0 on invalid arguments. */
size_t convrot_packed_bytes_w4a8_group(int64_t N, int64_t K, int group);

/* Workspace bytes for convrot_linear_w4a8 at this shape (scratch, like convrot_workspace_bytes);
 * 0 on invalid arguments (M outside [0, CONVROT_W4A8_MAX_M], K not a positive multiple of 128). */
size_t convrot_workspace_bytes_w4a8(int64_t M, int64_t N, int64_t K);

/*
 * Integer core without scales, for exactness checks: acc int32 [M, N] = xq . wq^T (same kernels
 * and M-based dispatch as convrot_linear; workspace unused, may be NULL).
 */
int convrot_gemm_i8_i32(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K, int32_t *acc,
                        void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * W4A4 integer core without scales: acc int32 [M, N] = sum_k cx[m,k] * cw[n,k] over packed codes
 * (same kernels as convrot_linear_w4a4; workspace of convrot_workspace_bytes(M, N, K, 4) bytes).
 */
int convrot_gemm_i4_i32(const uint8_t *xq, const uint8_t *wq, int64_t M, int64_t N, int64_t K, int32_t *acc,
                        void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Rotation group for a layer under the converter's dynamic mode: the largest group compatible
 * with the layer, capped by the configured size ("minimax-h3-nvfp4-convrot核心原理", section 四,
 * detail 3: --dynamic-convrot with --convrot-group-size 256).  Returns the largest power of two
 * <= max_group dividing K (256 for K = 5120 or 5376, 128 for the K = 2688 adaln projection), or
 * 0 when K <= 0 or max_group is not a power of two in [1, 256].  Pass the result as `group` to
 * convrot_prepare_weight, convrot_quantize_act, convrot_linear and, for 128 or 256,
 * convrot_linear_w4a4 and convrot_linear_w4a8 (the W4A4 and W4A8 paths take 256 or 128).
 */
int convrot_dynamic_group(int64_t K, int max_group);

/* Description of the last non-OK status returned on the calling thread ("" if none). */
const char *convrot_last_error(void);

/* Static name of a status code. */
const char *convrot_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_H */
