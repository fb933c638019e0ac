// rotate_quant.hip -- fused ConvRot rotate + quantize (gfx950).
//
// One pass over a row-major [rows, K] bf16/fp32 matrix: each row is rotated by the grouped
// Hadamard R = blockdiag(H_g / sqrt(g)) along K and quantized symmetrically with round to
// nearest even ("minimax-h3-nvfp4-convrot核心原理", section 四: weights pre-rotated by a
// fixed-group Hadamard before INT8 quantization; section 五: W4A4 rotates both operands and
// quantizes to 4 bits with RTN).
//   BITS = 8: one fp32 scale per row = max|rotated row| / 127 (weights: per output channel,
//             the row-wise scaling of the converter; activations: per token, at run time).
//   BITS = 4: one fp16 scale per (row, 256-channel group) = max|group| / 7, stored group-major
//             ([K/256, rows]); two codes per byte with the even channel in the low nibble.
// The same kernel prepares weights (rows = N) and quantizes activations (rows = M).
//
// Data layout in registers.  A row is cut into "slots" of 256 consecutive channels.  Inside a
// wavefront, lane bits 4:2 select one of 8 slots and the 8 lanes of a slot hold its 256
// values as 4 chunks x 8 channels each:
//     channel bits 2:0 -> element inside a chunk (one 16-byte bf16 load = 8 channels)
//     channel bits 4:3 -> lane bits 1:0   (butterfly partners reached with DPP quad_perm)
//     channel bit  5   -> lane bit 5      (moved into a register with v_permlane32_swap)
//     channel bits 7:6 -> chunk index r   (registers)
// so the 8-stage fast Walsh-Hadamard transform runs 6 stages in registers and 2 across lanes
// with no LDS traffic.  Each load instruction reads 128 contiguous bytes per slot.  The whole
// row stays in registers until its absmax is known, so HBM is read exactly once.
#include "device_common.hpp"
#include "launchers.hpp"

namespace convrot {

struct RQParams {
    const void *x;
    void *q;
    void *scale;
    int64_t rows;
    int K;
    int slots_per_row;   // ceil(K / 256)
    int rows_per_wg;     // rows handled by one workgroup (<= 64)
    int log2g;           // rotation group = 2^log2g channels (0..8)
    float cg;            // 1/sqrt(g) in fp32
};

__device__ __forceinline__ void bfly(float &a, float &b)
{
    const float s = a + b;
    b = a - b;
    a = s;
}

template <bool F32IN, int BITS, int SETS>
__global__ void __launch_bounds__(1024) rotate_quant_kernel(RQParams p)
{
    __shared__ unsigned smax[64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwave = blockDim.x >> 6;
    const int qd = lane & 3, h = lane >> 5, sl = (lane >> 2) & 7;
    if (threadIdx.x < 64) smax[threadIdx.x] = 0u;

    float v[SETS][4][8];
    int rr[SETS], jj[SETS];
    bool ok[SETS];
    int64_t rowv[SETS];

#pragma unroll
    for (int s = 0; s < SETS; ++s) {
        const int slot = (s * nwave + wave) * 8 + sl;
        rr[s] = slot / p.slots_per_row;
        jj[s] = slot - rr[s] * p.slots_per_row;
        rowv[s] = (int64_t)blockIdx.x * p.rows_per_wg + rr[s];
        ok[s] = rr[s] < p.rows_per_wg && rowv[s] < p.rows;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int k = 256 * jj[s] + 64 * r + 32 * h + 8 * qd;
            if (ok[s] && k < p.K) {
                if constexpr (F32IN) {
                    const v4f *src = reinterpret_cast<const v4f *>(
                        static_cast<const float *>(p.x) + rowv[s] * (int64_t)p.K + k);
                    const v4f a = __builtin_nontemporal_load(src);
                    const v4f b = __builtin_nontemporal_load(src + 1);
                    v[s][r][0] = a.x; v[s][r][1] = a.y; v[s][r][2] = a.z; v[s][r][3] = a.w;
                    v[s][r][4] = b.x; v[s][r][5] = b.y; v[s][r][6] = b.z; v[s][r][7] = b.w;
                } else {
                    const v4u *src = reinterpret_cast<const v4u *>(
                        static_cast<const uint16_t *>(p.x) + rowv[s] * (int64_t)p.K + k);
                    const v4u a = __builtin_nontemporal_load(src);
                    v[s][r][0] = bf16lo_to_f32(a.x); v[s][r][1] = bf16hi_to_f32(a.x);
                    v[s][r][2] = bf16lo_to_f32(a.y); v[s][r][3] = bf16hi_to_f32(a.y);
                    v[s][r][4] = bf16lo_to_f32(a.z); v[s][r][5] = bf16hi_to_f32(a.z);
                    v[s][r][6] = bf16lo_to_f32(a.w); v[s][r][7] = bf16hi_to_f32(a.w);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[s][r][e] = 0.0f;
            }
        }
    }

    // ---- unnormalised Walsh-Hadamard butterflies on channel bits < log2g (uniform branches)
    const int lg = p.log2g;
#pragma unroll
    for (int s = 0; s < SETS; ++s) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int b = 0; b < 3; ++b) {
                if (lg > b) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (!(e & (1 << b))) bfly(v[s][r][e], v[s][r][e | (1 << b)]);
                }
            }
        }
        // channel bits 3 and 4: partner is lane ^ 1 / lane ^ 2.  The lower lane keeps a + b,
        // the upper lane keeps a - b:  out = partner + c * self with c = -1 on the upper lane.
        if (lg > 3) {
            const float c = (qd & 1) ? -1.0f : 1.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int e = 0; e < 8; ++e) v[s][r][e] = __builtin_fmaf(v[s][r][e], c, dpp_xor1(v[s][r][e]));
        }
        if (lg > 4) {
            const float c = (qd & 2) ? -1.0f : 1.0f;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int e = 0; e < 8; ++e) v[s][r][e] = __builtin_fmaf(v[s][r][e], c, dpp_xor2(v[s][r][e]));
        }
        // channel bits 6 and 7: chunk registers
        if (lg > 6) {
#pragma unroll
            for (int e = 0; e < 8; ++e) { bfly(v[s][0][e], v[s][1][e]); bfly(v[s][2][e], v[s][3][e]); }
        }
        if (lg > 7) {
#pragma unroll
            for (int e = 0; e < 8; ++e) { bfly(v[s][0][e], v[s][2][e]); bfly(v[s][1][e], v[s][3][e]); }
        }
        // channel bit 5: swap it with chunk bit 0 (channel bit 6) between lane halves, then
        // butterfly in registers.  Afterwards v[s][2*r1 + c5][e] holds channel bit 5 = c5 and
        // channel bit 6 = lane bit 5.
        if (lg > 5) {
#pragma unroll
            for (int r1 = 0; r1 < 2; ++r1)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    swap32f(v[s][2 * r1][e], v[s][2 * r1 + 1][e]);
                    bfly(v[s][2 * r1][e], v[s][2 * r1 + 1][e]);
                }
        }
    }

    // ---- absmax: per slot over its 8 lanes (lane bits 0, 1 and 5)
    float m[SETS];
#pragma unroll
    for (int s = 0; s < SETS; ++s) {
        float a = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) a = __builtin_fmaxf(a, __builtin_fabsf(v[s][r][e]));
        a = __builtin_fmaxf(a, dpp_xor1(a));
        a = __builtin_fmaxf(a, dpp_xor2(a));
        uint32_t lo = __float_as_uint(a), hi = lo;
        swap32(lo, hi);
        m[s] = __builtin_fmaxf(__uint_as_float(lo), __uint_as_float(hi));
    }

    float mult[SETS];
    if constexpr (BITS == 8) {
        // row absmax across slots/waves through LDS (non-negative float bits order like uints)
        __syncthreads();
#pragma unroll
        for (int s = 0; s < SETS; ++s)
            if (ok[s] && qd == 0 && h == 0) atomicMax(&smax[rr[s]], __float_as_uint(m[s]));
        __syncthreads();
#pragma unroll
        for (int s = 0; s < SETS; ++s) {
            const float amax = __uint_as_float(smax[rr[s] < 64 ? rr[s] : 63]);
            const float sc = (amax * p.cg) / 127.0f;
            mult[s] = sc > 0.0f ? p.cg / sc : 0.0f;
            if (ok[s] && jj[s] == 0 && qd == 0 && h == 0) static_cast<float *>(p.scale)[rowv[s]] = sc;
        }
    } else {
        // one fp16 scale per 256-channel group (= slot)
#pragma unroll
        for (int s = 0; s < SETS; ++s) {
            const __half sh = __float2half_rn((m[s] * p.cg) / 7.0f);
            const float sc = __half2float(sh);
            mult[s] = sc > 0.0f ? p.cg / sc : 0.0f;
            if (ok[s] && qd == 0 && h == 0)
                static_cast<__half *>(p.scale)[(int64_t)jj[s] * p.rows + rowv[s]] = sh;
        }
    }

    // ---- codes, back to the load layout, store
#pragma unroll
    for (int s = 0; s < SETS; ++s) {
        if constexpr (BITS == 8) {
            uint32_t c[4][2];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint32_t t[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) t[e] = rne_bits(v[s][r][e], mult[s]);
                c[r][0] = pack4_i8(t[0], t[1], t[2], t[3]);
                c[r][1] = pack4_i8(t[4], t[5], t[6], t[7]);
            }
            if (lg > 5) {
#pragma unroll
                for (int r1 = 0; r1 < 2; ++r1) { swap32(c[2 * r1][0], c[2 * r1 + 1][0]); swap32(c[2 * r1][1], c[2 * r1 + 1][1]); }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int k = 256 * jj[s] + 64 * r + 32 * h + 8 * qd;
                if (ok[s] && k < p.K) {
                    uint2 *dst = reinterpret_cast<uint2 *>(static_cast<int8_t *>(p.q) + rowv[s] * (int64_t)p.K + k);
                    *dst = make_uint2(c[r][0], c[r][1]);
                }
            }
        } else {
            uint32_t c[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint32_t t[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) t[e] = rne_bits(v[s][r][e], mult[s]);
                c[r] = pack8_i4(t);
            }
            if (lg > 5) {
                swap32(c[0], c[1]);
                swap32(c[2], c[3]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int k = 256 * jj[s] + 64 * r + 32 * h + 8 * qd;
                if (ok[s] && k < p.K)
                    *reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(p.q) + rowv[s] * (int64_t)(p.K / 2) + k / 2) = c[r];
            }
        }
    }
}

// Host-side launch geometry: rows per workgroup and wavefronts per workgroup so that the
// 8 slots per wavefront are used as fully as possible (<= 16 wavefronts, <= 64 rows).
static void rq_geometry(int64_t rows, int K, int &rows_per_wg, int &waves, int &sets)
{
    const int G = (K + 255) / 256;
    sets = G <= 128 ? 1 : (G <= 256 ? 2 : 4);
    if (sets > 1) { rows_per_wg = 1; waves = (G + 8 * sets - 1) / (8 * sets); return; }
    double best = -1.0;
    rows_per_wg = 1;
    waves = (G + 7) / 8;
    for (int R = 1; R <= 64; ++R) {
        const int W = (R * G + 7) / 8;
        if (W > 16) break;
        if (R > rows && R > 1) break;
        double eff = (double)(R * G) / (8.0 * W);
        // prefer full slots, then 4..8 wavefronts per workgroup
        double score = eff - (W < 4 ? 0.02 * (4 - W) : 0.0) - (W > 8 ? 0.005 * (W - 8) : 0.0);
        if (score > best + 1e-9) { best = score; rows_per_wg = R; waves = W; }
    }
}

hipError_t launch_rotate_quant(const void *x, bool x_f32, int64_t rows, int K, int log2g, int bits, void *q,
                               void *scale, hipStream_t stream)
{
    if (rows <= 0) return hipSuccess;
    int R, W, S;
    rq_geometry(rows, K, R, W, S);
    RQParams p;
    p.x = x;
    p.q = q;
    p.scale = scale;
    p.rows = rows;
    p.K = K;
    p.slots_per_row = (K + 255) / 256;
    p.rows_per_wg = R;
    p.log2g = log2g;
    p.cg = (float)(1.0 / __builtin_sqrt((double)(1 << log2g)));
    const dim3 grid((unsigned)((rows + R - 1) / R)), block(64 * W);
#define RQ_LAUNCH(F32, B, SS) hipLaunchKernelGGL((rotate_quant_kernel<F32, B, SS>), grid, block, 0, stream, p)
#define RQ_SETS(F32, B)                  \
    do {                                 \
        if (S == 1) RQ_LAUNCH(F32, B, 1); \
        else if (S == 2) RQ_LAUNCH(F32, B, 2); \
        else RQ_LAUNCH(F32, B, 4);       \
    } while (0)
    if (x_f32) {
        if (bits == 8) RQ_SETS(true, 8); else RQ_SETS(true, 4);
    } else {
        if (bits == 8) RQ_SETS(false, 8); else RQ_SETS(false, 4);
    }
#undef RQ_SETS
#undef RQ_LAUNCH
    return hipGetLastError();
}

} // namespace convrot
