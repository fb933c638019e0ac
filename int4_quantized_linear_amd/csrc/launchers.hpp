// launchers.hpp -- internal host launchers of the ConvRot HIP kernels (not the public ABI).
// Every launcher assumes its arguments were validated by the C-ABI layer and only returns
// the launch status.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convrot {

// Rotate rows of x (bf16 or fp32, [rows, K]) by the grouped Hadamard and quantize:
// bits 8 -> q int8 [rows, K], scale fp32 [rows]; bits 4 -> q uint8 [rows, K/2], scale fp16 [rows, K/256].
hipError_t launch_rotate_quant(const void *x, bool x_f32, int64_t rows, int K, int log2g, int bits, void *q,
                               void *scale, hipStream_t stream);
// The INT4 case (log2g 7 or 8, K % 128 == 0) written straight as the FP6 tiles of the W4A4 GEMM:
// tiles of w4a4_tiled_bytes(rows, 0, K) bytes (rows padded to 32 with zero codes), scale as above.
hipError_t launch_rotate_quant_fp6(const void *x, bool x_f32, int64_t rows, int K, int log2g, uint8_t *tiles,
                                   void *scale, hipStream_t stream);

// Epilogue selector of the integer GEMM / GEMV kernels.
enum class Epi { Bf16 = 0, Int32 = 1 };

// y[M,N] = bf16(acc * sx[m] * sw[n] + bias[n])  or  acc32[M,N] = acc,   acc = xq . wq^T  (M > 16).
// part: optional scratch for the split-K tail (bf16 output only): when the tiles leave the last
// round of the persistent grid partly idle and part_bytes >= gemm_i8_split_bytes(M, N, K), the
// tail tiles are computed as K-slices whose int32 partial sums meet in `part`, then a second
// kernel sums them and applies the epilogue (bit-identical outputs).  part == nullptr: no split.
hipError_t launch_gemm_i8(const int8_t *xq, const int8_t *wq, const float *sx, const float *sw, const float *bias,
                          void *y, Epi epi, int64_t M, int64_t N, int K, void *part, size_t part_bytes,
                          hipStream_t stream);
// Bytes of `part` the split-K tail uses for this shape on the current device (0: no split).
size_t gemm_i8_split_bytes(int64_t M, int64_t N, int K);

// Same contraction for M <= 16 (weight streaming; K split among the wavefronts of a workgroup,
// no scratch memory).
hipError_t launch_gemv_i8(const int8_t *xq, const int8_t *wq, const float *sx, const float *sw, const float *bias,
                          void *y, Epi epi, int64_t M, int64_t N, int K, hipStream_t stream);

// W4A4: y = bf16(sum_g acc_g * sx[m,g] * sw[n,g] + bias[n]) with packed int4 operands and
// fp16 group scales (group = 256 or 128, K % group == 0, K >= 256), or the unscaled int32 total
// sum_k cx*cw (scales ignored).
// Both operands run through the FP6 tiles of launch_tile_w4a4: the tokens are re-encoded into
// the start of `ws` unless x_tiled says xq already holds their tiles (launch_rotate_quant_fp6),
// the weights after them unless w_tiled says wq does.  `ws` is scratch of
// w4a4_tiled_bytes(M, w_tiled ? 0 : N, K) bytes (16-byte aligned).
size_t w4a4_tiled_bytes(int64_t M, int64_t N, int K);
// Packed int4 rows [R, K/2] -> FP6 tiles (w4a4_tiled_bytes(R, 0, K) bytes), K % 128 == 0.
hipError_t launch_tile_w4a4(const uint8_t *q, int64_t R, int K, uint8_t *out, hipStream_t stream);
hipError_t launch_gemm_w4a4(const uint8_t *xq, bool x_tiled, const uint8_t *wq, bool w_tiled, const uint16_t *sx,
                            const uint16_t *sw, const float *bias, void *y, Epi epi, int64_t M, int64_t N, int K,
                            int group, void *ws, hipStream_t stream);

// W4A8 decode linear (M <= 16): y = bf16(sx[m] * sum_g sw[g,n] * (qx . cw over group g) + bias[n])
// with INT8 tokens and the weights in the W4A8 block layout (codes and fp16 group scales), made
// once by launch_pack_w4a8 from packed INT4 [N, K/2] and scales [K/group, N] (group 256, or 128
// with two scale sets per 256-channel block); N % 8 == 0.
// No scratch memory: K is split only among the wavefronts of one workgroup.
size_t w4a8_packed_bytes(int64_t N, int K, int group);
hipError_t launch_pack_w4a8(const uint8_t *wq, const uint16_t *sw, int64_t N, int K, int group, uint8_t *out,
                            hipStream_t stream);
int gemv_w4a8_waves(int64_t N, int K);
hipError_t launch_gemv_w4a8(const int8_t *xq, const float *sx, const uint8_t *wp, const float *bias, void *y,
                            int64_t M, int64_t N, int K, int group, hipStream_t stream);

} // namespace convrot
