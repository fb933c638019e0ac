// rotate_quant.hip -- fused ConvRot rotate + quantize (gfx950).
//
// One pass over a row-major [rows, K] bf16/fp32 matrix: each row is rotated by the grouped
// Hadamard R = blockdiag(H_g / sqrt(g)) along K and quantized symmetrically with round to
// nearest even ("minimax-h3-nvfp4-convrot核心原理", section 四: weights pre-rotated by a
// fixed-group Hadamard before INT8 quantization; section 五: W4A4 rotates both operands and
// quantizes to 4 bits with RTN).
//   BITS = 8: one fp32 scale per row = max|rotated row| / 127 (weights: per output channel,
//             the row-wise scaling of the converter; activations: per token, at run time).
//   BITS = 4: one fp16 scale per (row, g-channel group) = max|group| / 7 with g = 256, or 128
//             for a width 256 does not divide (section 四, detail 3, dynamic group), stored
//             group-major ([K/g, rows]); two codes per byte with the even channel in the low nibble.
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
    int rows_per_wg;     // rows handled by one workgroup per iteration (<= 64)
    int ngroups;         // ceil(rows / rows_per_wg)
    float cg;            // 1/sqrt(g) in fp32
    double root;         // sqrt(g) in fp64
};

constexpr uint32_t OOB = 0x80000000u;   // buffer offset past num_records: loads read 0, stores drop

__device__ __forceinline__ void bfly(float &a, float &b)
{
    const float s = a + b;
    b = a - b;
    a = s;
}

// Unnormalised Walsh-Hadamard transform of one slot held as 4 chunks x 8 values per lane (the
// register layout above), on channel bits < LG.  qd = lane & 3.
template <int LG>
__device__ __forceinline__ void fwht_slot(float (&v)[4][8], int qd)
{
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int b = 0; b < 3; ++b) {
            if (LG > b) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (!(e & (1 << b))) bfly(v[r][e], v[r][e | (1 << b)]);
            }
        }
    }
    // channel bits 6 and 7: chunk registers
    if constexpr (LG > 6) {
#pragma unroll
        for (int e = 0; e < 8; ++e) { bfly(v[0][e], v[1][e]); bfly(v[2][e], v[3][e]); }
    }
    if constexpr (LG > 7) {
#pragma unroll
        for (int e = 0; e < 8; ++e) { bfly(v[0][e], v[2][e]); bfly(v[1][e], v[3][e]); }
    }
    // channel bit 5: swap it with chunk bit 0 (channel bit 6) between lane halves, then butterfly
    // in registers.  Afterwards v[2*r1 + c5][e] holds channel bit 5 = c5 and channel bit 6 =
    // lane bit 5.
    if constexpr (LG > 5) {
#pragma unroll
        for (int r1 = 0; r1 < 2; ++r1)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                swap32f(v[2 * r1][e], v[2 * r1 + 1][e]);
                bfly(v[2 * r1][e], v[2 * r1 + 1][e]);
            }
    }
    // channel bits 3 and 4, last: partner is lane ^ 1 / lane ^ 2.  Each stage is one
    // v_fmac_f32_dpp per value: self + partner * c, c = +1 on the lower lane (a + b, correct) and
    // -1 on the upper lane (b - a, the negated result).  Running the two lane stages after all
    // others keeps that sign error out of every other butterfly: the final value of a lane is off
    // by the sign (-1)^(bit0 ^ bit1) of its quad position, which is folded into the quantization
    // multiplier and does not change |v|.
    if constexpr (LG > 3) {
        const float c = (qd & 1) ? -1.0f : 1.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) fmac_dpp8_xor1_(v[r], c);
    }
    if constexpr (LG > 4) {
        const float c = (qd & 2) ? -1.0f : 1.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) fmac_dpp8_xor2_(v[r], c);
    }
}

// LG = log2 of the rotation group (0..8), a template parameter so that the butterfly stages are
// straight-line code.  All global accesses are buffer instructions whose out-of-range lanes get
// an out-of-bounds offset (loads return 0, stores are dropped): no branches around them, so the
// loads of a wavefront are all in flight together.
//
// Persistent: a workgroup walks row groups blockIdx.x, blockIdx.x + gridDim.x, ... and issues
// the raw loads of its next row group before it transforms the current one, so HBM reads stay
// in flight while the VALU works (without this, all waves would load, then all compute).
template <bool F32IN, int BITS, int SETS, int LG>
__global__ void __launch_bounds__(1024) rotate_quant_kernel(RQParams p)
{
    __shared__ unsigned smax[2][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwave = blockDim.x >> 6;
    const int qd = lane & 3, h = lane >> 5, sl = (lane >> 2) & 7;
    if (threadIdx.x < 64) smax[0][threadIdx.x] = 0u;

    constexpr int ES = F32IN ? 4 : 2;                       // input element bytes
    constexpr int NL = F32IN ? 2 : 1;                       // 16-byte loads per chunk
    const int K = p.K;
    const int R = p.rows_per_wg;

    // Static slot geometry: slot -> (row within the group, 256-channel block); element offset
    // of each chunk inside the row group, or OOB for slots/channels past the row or the group.
    int rr[SETS], jj[SETS];
    uint32_t kbase[SETS][4];
#pragma unroll
    for (int s = 0; s < SETS; ++s) {
        const int slot = (s * nwave + wave) * 8 + sl;
        rr[s] = slot / p.slots_per_row;
        jj[s] = slot - rr[s] * p.slots_per_row;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int k = 256 * jj[s] + 64 * r + 32 * h + 8 * qd;
            kbase[s][r] = (rr[s] < R && k < K) ? (uint32_t)(rr[s] * K + k) : OOB;
        }
    }

    v4u raw[SETS][4][NL];
    auto issue = [&](int it) {
        const int64_t row0 = (int64_t)it * R;
        const int nrows = (int)(p.rows - row0 < R ? p.rows - row0 : R);
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(static_cast<const uint8_t *>(p.x) + row0 * K * ES), (short)0, nrows * K * ES,
            0x00020000);
#pragma unroll
        for (int s = 0; s < SETS; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int l = 0; l < NL; ++l) {
                    // rows past the end lie past num_records: they read zeros.  Read once:
                    // nontemporal (aux bit 1).
                    const uint32_t o = kbase[s][r] == OOB ? OOB : kbase[s][r] * ES + 16 * l;
                    raw[s][r][l] = __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, 2);
                }
    };

    // Prefetching holds a second copy of the raw row data: only for SETS == 1 (K <= 32768); the
    // wider rows would not fit the registers of a 1024-thread workgroup.
    constexpr bool PF = SETS == 1;
    int it = blockIdx.x;
    int par = 0;
    if (PF && it < p.ngroups) issue(it);
    for (; it < p.ngroups; it += gridDim.x, par ^= 1) {
        if constexpr (!PF) issue(it);
        const int64_t row0 = (int64_t)it * R;
        const int nrows = (int)(p.rows - row0 < R ? p.rows - row0 : R);
        float v[SETS][4][8];
#pragma unroll
        for (int s = 0; s < SETS; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (F32IN) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[s][r][e] = __uint_as_float(raw[s][r][e >> 2][e & 3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[s][r][2 * e] = bf16lo_to_f32(raw[s][r][0][e]);
                        v[s][r][2 * e + 1] = bf16hi_to_f32(raw[s][r][0][e]);
                    }
                }
            }
        if (PF && it + (int)gridDim.x < p.ngroups) issue(it + gridDim.x);   // prefetch the next group
        bool ok[SETS];
#pragma unroll
        for (int s = 0; s < SETS; ++s) ok[s] = rr[s] < nrows;

        // ---- unnormalised Walsh-Hadamard butterflies on channel bits < LG
#pragma unroll
        for (int s = 0; s < SETS; ++s) fwht_slot<LG>(v[s], qd);

        // ---- absmax: per slot over its 8 lanes (lane bits 0, 1 and 5); for INT4 with 128-channel
        // groups, per half slot: channel bit 7 is the register pair (registers 0, 1 | 2, 3)
        constexpr int HS = (BITS == 4 && LG == 7) ? 2 : 1;   // scale groups per slot
        float m[SETS][HS];
#pragma unroll
        for (int s = 0; s < SETS; ++s) {
#pragma unroll
            for (int hs = 0; hs < HS; ++hs) {
                float a = 0.0f;
#pragma unroll
                for (int r = hs * (4 / HS); r < (hs + 1) * (4 / HS); ++r)
#pragma unroll
                    for (int e = 0; e < 8; ++e) a = __builtin_fmaxf(a, __builtin_fabsf(v[s][r][e]));
                a = __builtin_fmaxf(a, dpp_xor1(a));
                a = __builtin_fmaxf(a, dpp_xor2(a));
                uint32_t lo = __float_as_uint(a), hi = lo;
                swap32(lo, hi);
                m[s][hs] = __builtin_fmaxf(__uint_as_float(lo), __uint_as_float(hi));
            }
        }

        // fp32 of a normalised maximum, from the maximum of the unnormalised sums: for even LG,
        // 1/sqrt(g) is a power of two and the product is exact; otherwise the division by sqrt(g)
        // runs in fp64 and is rounded once to fp32, which is the fp32 rounding of the
        // normalised value whenever the unnormalised fp32 sum is exact
        auto normalised = [&](float m_u) -> float {
            if constexpr (LG % 2 == 0) return m_u * p.cg;
            else return (float)((double)m_u / p.root);
        };
        // sign left on this lane's values by the lane-exchange butterflies
        const float lsign = (((LG > 3 ? qd : 0) ^ (LG > 4 ? qd >> 1 : 0)) & 1) ? -1.0f : 1.0f;
        float mult[SETS][HS];
        if constexpr (BITS == 8) {
            // row absmax across slots/waves through LDS (non-negative float bits order like uints).
            // smax[par] was cleared before the previous iteration's first barrier; the other
            // buffer, last read before this barrier, is cleared for the next iteration.
            __syncthreads();
            if (threadIdx.x < 64) smax[par ^ 1][threadIdx.x] = 0u;
#pragma unroll
            for (int s = 0; s < SETS; ++s)
                if (ok[s] && qd == 0 && h == 0) atomicMax(&smax[par][rr[s]], __float_as_uint(m[s][0]));
            __syncthreads();
#pragma unroll
            for (int s = 0; s < SETS; ++s) {
                const float amax = __uint_as_float(smax[par][rr[s] < 64 ? rr[s] : 63]);
                const float sc = normalised(amax) / 127.0f;
                mult[s][0] = sc > 0.0f ? lsign * (p.cg / sc) : 0.0f;
                if (ok[s] && jj[s] == 0 && qd == 0 && h == 0) static_cast<float *>(p.scale)[row0 + rr[s]] = sc;
            }
        } else {
            // one fp16 scale per g-channel group: the slot (g = 256) or each half of it (g = 128);
            // a half slot past the end of K (K % 256 == 128) is padding and stores no scale
#pragma unroll
            for (int s = 0; s < SETS; ++s)
#pragma unroll
                for (int hs = 0; hs < HS; ++hs) {
                    // one rounding to fp16 from the exact quotient (no double rounding through fp32)
                    const __half sh = f16_quotient_rne(normalised(m[s][hs]), 7.0f);
                    const float sc = __half2float(sh);
                    mult[s][hs] = sc > 0.0f ? lsign * (p.cg / sc) : 0.0f;
                    const int64_t grp = (int64_t)jj[s] * HS + hs;
                    if (ok[s] && qd == 0 && h == 0 && grp * (256 / HS) < K)
                        static_cast<__half *>(p.scale)[grp * p.rows + row0 + rr[s]] = sh;
                }
        }

        // ---- codes, back to the load layout, store (rows past the group's end lie past
        // num_records and are dropped)
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            static_cast<uint8_t *>(p.q) + (BITS == 8 ? row0 * K : row0 * (K / 2)), (short)0,
            BITS == 8 ? nrows * K : nrows * (K / 2), 0x00020000);
#pragma unroll
        for (int s = 0; s < SETS; ++s) {
            if constexpr (BITS == 8) {
                uint32_t c[4][2];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uint32_t t[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) t[e] = rne_bits(v[s][r][e], mult[s][0]);
                    c[r][0] = pack4_i8(t[0], t[1], t[2], t[3]);
                    c[r][1] = pack4_i8(t[4], t[5], t[6], t[7]);
                }
                if constexpr (LG > 5) {
#pragma unroll
                    for (int r1 = 0; r1 < 2; ++r1) { swap32(c[2 * r1][0], c[2 * r1 + 1][0]); swap32(c[2 * r1][1], c[2 * r1 + 1][1]); }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    __builtin_amdgcn_raw_buffer_store_b64(v2u{c[r][0], c[r][1]}, rq, kbase[s][r], 0, 0);
            } else {
                uint32_t c[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uint32_t t[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) t[e] = rne_bits(v[s][r][e], mult[s][r / (4 / HS)]);
                    c[r] = pack8_i4(t);
                }
                if constexpr (LG > 5) {
                    swap32(c[0], c[1]);
                    swap32(c[2], c[3]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    __builtin_amdgcn_raw_buffer_store_b32(c[r], rq, kbase[s][r] == OOB ? OOB : kbase[s][r] / 2, 0, 0);
            }
        }
    }
}

constexpr int RQ_WAVES_PER_CU = 16;

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

template <bool F32, int B, int SS>
static void rq_launch_lg(int log2g, dim3 grid, dim3 block, hipStream_t stream, const RQParams &p)
{
    switch (log2g) {
    case 0: hipLaunchKernelGGL((rotate_quant_kernel<F32, B, SS, 0>), grid, block, 0, stream, p); break;
    case 1: hipLaunchKernelGGL((rotate_quant_kernel<F32, B, SS, 1>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((rotate_quant_kernel<F32, B, SS, 2>), grid, block, 0, stream, p); break;
    case 3: hipLaunchKernelGGL((rotate_quant_kernel<F32, B, SS, 3>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((rotate_quant_kernel<F32, B, SS, 4>), grid, block, 0, stream, p); break;
    case 5: hipLaunchKernelGGL((rotate_quant_kernel<F32, B, SS, 5>), grid, block, 0, stream, p); break;
    case 6: hipLaunchKernelGGL((rotate_quant_kernel<F32, B, SS, 6>), grid, block, 0, stream, p); break;
    case 7: hipLaunchKernelGGL((rotate_quant_kernel<F32, B, SS, 7>), grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL((rotate_quant_kernel<F32, B, SS, 8>), grid, block, 0, stream, p); break;
    }
}

template <bool F32, int B>
static void rq_launch(int sets, int log2g, dim3 grid, dim3 block, hipStream_t stream, const RQParams &p)
{
    if (sets == 1) rq_launch_lg<F32, B, 1>(log2g, grid, block, stream, p);
    else if (sets == 2) rq_launch_lg<F32, B, 2>(log2g, grid, block, stream, p);
    else rq_launch_lg<F32, B, 4>(log2g, grid, block, stream, p);
}

// INT4: the scale group is the rotation group, 256 or 128 channels (checked by the C-ABI layer)
template <bool F32, int LG>
static void rq_launch_i4(int sets, dim3 grid, dim3 block, hipStream_t stream, const RQParams &p)
{
    if (sets == 1) hipLaunchKernelGGL((rotate_quant_kernel<F32, 4, 1, LG>), grid, block, 0, stream, p);
    else if (sets == 2) hipLaunchKernelGGL((rotate_quant_kernel<F32, 4, 2, LG>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((rotate_quant_kernel<F32, 4, 4, LG>), grid, block, 0, stream, p);
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
    p.ngroups = (int)((rows + R - 1) / R);
    p.root = __builtin_sqrt((double)(1 << log2g));
    p.cg = (float)(1.0 / p.root);
    static const int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            n = 256;
        return n > 0 ? n : 256;
    }();
    // persistent grid: about RQ_WAVES_PER_CU resident wavefronts per CU, each workgroup looping
    const int per_cu = RQ_WAVES_PER_CU / W > 1 ? RQ_WAVES_PER_CU / W : 1;
    const int64_t g = (int64_t)cus * per_cu < p.ngroups ? (int64_t)cus * per_cu : p.ngroups;
    const dim3 grid((unsigned)g), block(64 * W);
    if (bits == 4 && log2g != 7 && log2g != 8) return hipErrorInvalidValue;
    if (x_f32) {
        if (bits == 8) rq_launch<true, 8>(S, log2g, grid, block, stream, p);
        else if (log2g == 8) rq_launch_i4<true, 8>(S, grid, block, stream, p);
        else rq_launch_i4<true, 7>(S, grid, block, stream, p);
    } else {
        if (bits == 8) rq_launch<false, 8>(S, log2g, grid, block, stream, p);
        else if (log2g == 8) rq_launch_i4<false, 8>(S, grid, block, stream, p);
        else rq_launch_i4<false, 7>(S, grid, block, stream, p);
    }
    return hipGetLastError();
}

} // namespace convrot
