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
// The same kernel prepares weights (rows = N) and quantizes activations (rows = M).  A second
// kernel below (rotate_quant_fp6_kernel) computes the BITS = 4 codes and scales of activations the
// same way and writes the codes straight in the FP6 matrix-core layout of the W4A4 GEMM.
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
    double rinv;         // 1/sqrt(g) in fp64
    float cg_lo;         // fp32(1/sqrt(g) - cg): with cg, 1/sqrt(g) to ~48 bits
};

// The code is rint of the correctly rounded fp32 quotient of the normalised value v = fp32(vu /
// sqrt(g)) by the stored scale s, as its definition states, not of a product with a rounded
// reciprocal: rotated sums of bf16 values often carry few significant bits, so exact half-integer
// quotients are common (3-5e-4 of the codes of N(0, 0.02) bf16 weight rows at g = 1 or 2, and of
// small-integer activations at g = 256) and a rounded reciprocal breaks those ties either way.
//
// Quotient: m = RN(1 / s), q0 = RN(v m) is within an ulp of v / s, the remainder v - q0 s is
// exact in one fma, and one correction step q0 + (v - q0 s) m rounds correctly (Markstein's
// theorem).  The sign the lane-exchange butterflies left on this lane's values goes into both
// factors, and for even log2 g so does 1/sqrt(g) = cg, a power of two (a = sign cg m, b = s /
// (sign cg): exact scalings), so the unnormalised sum vu enters directly.  For odd log2 g, the
// normalised magnitude is vu cg + vu cg_lo in one fma, the correctly rounded product unless
// vu / sqrt(g) lies within ~2^-47 of a rounding midpoint, with a = sign m, b = sign s.  s == 0
// comes with a = b = 0 and vu == 0: the code is 0.
struct QuotientRN {
    float a, b;
};

template <int LG>
__device__ __forceinline__ QuotientRN quotient_consts(float s, float sign, float cg)
{
    const float m = s > 0.0f ? 1.0f / s : 0.0f;
    if constexpr (LG % 2 == 0) return {m * (sign * cg), s > 0.0f ? s / (sign * cg) : 0.0f};
    else return {sign * m, sign * s};
}

// the scale s back from the constants (exact)
template <int LG>
__device__ __forceinline__ float quotient_scale(QuotientRN k, float cg)
{
    return LG % 2 == 0 ? __builtin_fabsf(k.b) * cg : __builtin_fabsf(k.b);
}

// fp32 of the quotient (before rint) for an unnormalised rotated value vu
template <int LG>
__device__ __forceinline__ float quotient_rn(float vu, QuotientRN k, float cg, float cg_lo)
{
    float v = vu;
    if constexpr (LG % 2 != 0) v = __builtin_fmaf(vu, cg, vu * cg_lo);
    const float q0 = v * k.a;
    const float r = __builtin_fmaf(-q0, k.b, v);
    return __builtin_fmaf(r, k.a, q0);
}

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
// Persistent: a workgroup walks row groups blockIdx.x, blockIdx.x + gridDim.x, ...  Two
// workgroups share a CU (the grid holds about RQ_WAVES_PER_CU wavefronts per CU), so one's loads
// are in flight while the other transforms; carrying the next row group's loads in registers
// instead costs enough registers to halve that and is slower.
template <bool F32IN, int BITS, int SETS, int LG>
__device__ __forceinline__ void rotate_quant_body(const RQParams &p)
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

    int it = blockIdx.x;
    int par = 0;
    for (; it < p.ngroups; it += gridDim.x, par ^= 1) {
        issue(it);
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
        QuotientRN qk[SETS][HS];
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
                qk[s][0] = quotient_consts<LG>(sc, lsign, p.cg);
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
                    qk[s][hs] = quotient_consts<LG>(sc, lsign, p.cg);
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
                QuotientRN k = qk[s][0];
                // the row's fp32 scale, exactly, from the constants; below 2^-100, 1/s can
                // overflow, so such rows (numerically zero: max |v| < 127 * 2^-100) take v and s
                // scaled by 2^64, which is exact and leaves every quotient as it is
                const float sc = quotient_scale<LG>(k, p.cg);
                const bool tiny = sc > 0.0f && sc < 0x1p-100f;
                if (__builtin_amdgcn_ballot_w64(tiny) != 0 && tiny) {
                    k = quotient_consts<LG>(sc * 0x1p64f, lsign, p.cg);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[s][r][e] *= 0x1p64f;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uint32_t t[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) t[e] = rne_bits(quotient_rn<LG>(v[s][r][e], k, p.cg, p.cg_lo), 1.0f);
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
                    for (int e = 0; e < 8; ++e)
                        t[e] = rne_bits(quotient_rn<LG>(v[s][r][e], qk[s][r / (4 / HS)], p.cg, p.cg_lo), 1.0f);
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


// One row slot set per wavefront (K <= 32768): two 16-wavefront workgroups per CU, so at most 64
// VGPRs (8 wavefronts per SIMD).  More sets hold more of the row in registers and run with fewer.
template <bool F32IN, int BITS, int SETS, int LG>
__global__ void __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(8))) rotate_quant_kernel(RQParams p)
{
    rotate_quant_body<F32IN, BITS, SETS, LG>(p);
}

template <bool F32IN, int BITS, int SETS, int LG>
__global__ void __launch_bounds__(1024) rotate_quant_wide_kernel(RQParams p)
{
    rotate_quant_body<F32IN, BITS, SETS, LG>(p);
}

// ---------------------------------------------------------------------------------------------
// INT4 straight into the FP6 tiles of the W4A4 GEMM.  Same rotation, scales and codes as the
// BITS = 4 kernel above (the 4-bit scale group is a slot or half a slot, so no reduction leaves
// a slot), but the codes are written as the E3M2 pieces the GEMM streams (gemm_w4a4.hip: per
// 32-row block and 64-channel K-step a 1536-byte piece; lane l = (row r = l % 32, half h = l / 32)
// owns the 32 codes at channels 64 ks + 32 h + s, 6 bits each at bit 6 s of a 24-byte string
// whose bytes 0..15 sit at 16 l and 16..23 at 1024 + 8 l; rows past the matrix are zeros).
//
// Work unit: one 32-row block x one 256-channel block, a 256-thread workgroup, so that all of a
// piece's cache lines are written by one CU.  Wavefront w takes rows 8 w .. 8 w + 7, one slot
// (row) per lane bits 4:2 and the in-slot layout of the kernel above.  After the butterflies, lane
// (qd, h) holds, in register r, 8 codes of K-step 4 j + r at s = 8 qd .. 8 qd + 7 of half h
// (once the lane halves are swapped back), i.e. 48 bits at bit 48 qd of lane string l.  One
// v_cvt_scalef32_2xpk16_bf6_f32 turns the lane's 32 integer-valued floats into 6 dwords of E3M2
// (position 2i from the first source's element i, 2i + 1 from the second's; scale 1: exact for
// integers up to 8 in magnitude), ordered so that dwords 0..2 hold registers 0 and 2 and dwords
// 3..5 registers 1 and 3: the swap of lane halves then runs on whole dwords.  Each lane stores its
// 48 bits of each K-step as one dword and one short.
//
// Rows from the matrix's end up to the next multiple of 32 read zeros (past num_records) and
// write zero codes; their scales are not stored.

struct RQ6Params {
    const void *x;
    uint8_t *tiles;      // [ceil(rows / 32)][K / 64][1536]
    __half *scale;       // [K / g, rows]
    int64_t rows;
    int K;
    int nblk;            // ceil(K / 256)
    float cg;
    float cg_lo;
    double root;
};

typedef unsigned v6u __attribute__((ext_vector_type(6)));

template <bool F32IN, int LG>
__global__ void __launch_bounds__(256) rotate_quant_fp6_kernel(RQ6Params p)
{
    constexpr int PIECE = 1536;
    constexpr int ES = F32IN ? 4 : 2;
    constexpr int NL = F32IN ? 2 : 1;
    constexpr int HS = LG == 7 ? 2 : 1;                    // scale groups per slot
    const int lane = threadIdx.x & 63;
    const int qd = lane & 3, h = lane >> 5, sl = (lane >> 2) & 7;
    const int rw = 8 * (threadIdx.x >> 6) + sl;           // row inside the 32-row block
    const int K = p.K, KS = K >> 6;
    const uint32_t u = blockIdx.x;
    const uint32_t rb = u / (uint32_t)p.nblk, j = u - rb * (uint32_t)p.nblk;
    const int64_t row0 = 32 * (int64_t)rb;
    const int nrows = (int)(p.rows - row0 < 32 ? p.rows - row0 : 32);

    // loads: 4 chunks of 8 channels (rows past the matrix lie past num_records and read zeros;
    // the second half of a 128-channel last block is out of range too)
    v4u raw[4][NL];
    {
        const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint8_t *>(static_cast<const uint8_t *>(p.x) + row0 * K * ES), (short)0, nrows * K * ES,
            0x00020000);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int k = 256 * (int)j + 64 * r + 32 * h + 8 * qd;
            const uint32_t o = (rw < nrows && k < K) ? (uint32_t)(rw * K + k) * ES : OOB;
#pragma unroll
            for (int q = 0; q < NL; ++q)
                raw[r][q] = __builtin_amdgcn_raw_buffer_load_b128(rx, o == OOB ? OOB : o + 16 * q, 0, 2);
        }
    }
    float v[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if constexpr (F32IN) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[r][e] = __uint_as_float(raw[r][e >> 2][e & 3]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[r][2 * e] = bf16lo_to_f32(raw[r][0][e]);
                v[r][2 * e + 1] = bf16hi_to_f32(raw[r][0][e]);
            }
        }
    }

    fwht_slot<LG>(v, qd);

    // per scale group: absmax over the slot's 8 lanes, fp16 scale, the quotient's constants (with
    // the sign the lane-exchange stages left on this lane); fp16 scales are >= 2^-24, so 1/s is finite
    const float lsign = ((qd ^ (qd >> 1)) & 1) ? -1.0f : 1.0f;
    QuotientRN qk[HS];
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) {
        float a = 0.0f;
#pragma unroll
        for (int r = hs * (4 / HS); r < (hs + 1) * (4 / HS); ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) a = __builtin_fmaxf(a, __builtin_fabsf(v[r][e]));
        a = __builtin_fmaxf(a, dpp_xor1(a));
        a = __builtin_fmaxf(a, dpp_xor2(a));
        uint32_t lo = __float_as_uint(a), hi = lo;
        swap32(lo, hi);
        a = __builtin_fmaxf(__uint_as_float(lo), __uint_as_float(hi));
        const float an = LG % 2 == 0 ? a * p.cg : (float)((double)a / p.root);
        const __half sh = f16_quotient_rne(an, 7.0f);
        const float sc = __half2float(sh);
        qk[hs] = quotient_consts<LG>(sc, lsign, p.cg);
        const int64_t grp = (int64_t)j * HS + hs;
        if (rw < nrows && qd == 0 && h == 0 && grp * (256 / HS) < K) p.scale[grp * p.rows + row0 + rw] = sh;
    }

    // integer-valued codes (rint of the correctly rounded quotient, as in the kernel above) in the conversion's source order:
    // output position 2i + b <- source b element i; positions 0..7 register 0, 8..15 register 2,
    // 16..23 register 1, 24..31 register 3
    v16f src[2];
#pragma unroll
    for (int pos = 0; pos < 32; ++pos) {
        const int r = (pos >> 4) | ((pos >> 2) & 2), e = pos & 7;
        src[pos & 1][pos >> 1] =
            (quotient_rn<LG>(v[r][e], qk[r / (4 / HS)], p.cg, p.cg_lo) + kMagicRound) - kMagicRound;
    }
    const v6u d = __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(src[0], src[1], 1.0f);
    uint32_t dw[6] = {d[0], d[1], d[2], d[3], d[4], d[5]};
    // lane halves back: afterwards dwords 0..2 hold K-steps 0 and 2, dwords 3..5 K-steps 1 and 3
#pragma unroll
    for (int i = 0; i < 3; ++i) swap32(dw[i], dw[i + 3]);

    // this lane's 6 bytes of each K-step's string (bytes 6 qd .. 6 qd + 5) as one dword and one
    // short; K-steps past K lie past num_records
    const uint32_t l = (uint32_t)rw + 32u * (uint32_t)h;
    const uint32_t o32 = qd == 0 ? 16u * l : qd == 1 ? 16u * l + 8u : qd == 2 ? 16u * l + 12u : 1028u + 8u * l;
    const uint32_t o16 = qd == 0 ? 16u * l + 4u : qd == 1 ? 16u * l + 6u : qd == 2 ? 1024u + 8u * l : 1026u + 8u * l;
    const bool odd = qd & 1;
    const int nks = KS - 4 * (int)j < 4 ? KS - 4 * (int)j : 4;
    const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
        p.tiles + ((int64_t)rb * KS + 4 * (int64_t)j) * PIECE, (short)0, nks * PIECE, 0x00020000);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        // the 48-bit string of K-step ks: low dword c0, high half c1 (low 16 bits)
        const uint32_t *b = dw + 3 * (ks & 1);
        const uint32_t c0 = ks < 2 ? b[0] : __builtin_amdgcn_alignbit(b[2], b[1], 16);
        const uint32_t c1 = ks < 2 ? b[1] : b[2] >> 16;
        const uint32_t w32 = odd ? __builtin_amdgcn_alignbit(c1, c0, 16) : c0;
        const uint32_t w16 = odd ? c0 : c1;
        __builtin_amdgcn_raw_buffer_store_b32(w32, rt, o32 + ks * PIECE, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)w16, rt, o16 + ks * PIECE, 0, 0);
    }
}

hipError_t launch_rotate_quant_fp6(const void *x, bool x_f32, int64_t rows, int K, int log2g, uint8_t *tiles,
                                   void *scale, hipStream_t stream)
{
    if (rows <= 0) return hipSuccess;
    if ((log2g != 7 && log2g != 8) || K % 128 || K < 128) return hipErrorInvalidValue;
    RQ6Params p;
    p.x = x;
    p.tiles = tiles;
    p.scale = static_cast<__half *>(scale);
    p.rows = rows;
    p.K = K;
    p.nblk = (K + 255) / 256;
    const int64_t units = ((rows + 31) / 32) * p.nblk;
    if (units >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    p.root = __builtin_sqrt((double)(1 << log2g));
    p.cg = (float)(1.0 / p.root);
    p.cg_lo = (float)(1.0 / p.root - (double)p.cg);
    // one workgroup per unit: ~40 resident wavefronts per CU at this kernel's register count (a
    // persistent grid with the next unit's loads in flight holds fewer and is slower)
    const dim3 grid((unsigned)units), block(256);
    if (x_f32) {
        if (log2g == 8) hipLaunchKernelGGL((rotate_quant_fp6_kernel<true, 8>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((rotate_quant_fp6_kernel<true, 7>), grid, block, 0, stream, p);
    } else {
        if (log2g == 8) hipLaunchKernelGGL((rotate_quant_fp6_kernel<false, 8>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((rotate_quant_fp6_kernel<false, 7>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

constexpr int RQ_WAVES_PER_CU = 32;

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

template <bool F32, int B, int SS, int LG>
static void rq_launch_one(dim3 grid, dim3 block, hipStream_t stream, const RQParams &p)
{
    if constexpr (SS == 1) hipLaunchKernelGGL((rotate_quant_kernel<F32, B, SS, LG>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((rotate_quant_wide_kernel<F32, B, SS, LG>), grid, block, 0, stream, p);
}

template <bool F32, int B, int SS>
static void rq_launch_lg(int log2g, dim3 grid, dim3 block, hipStream_t stream, const RQParams &p)
{
    switch (log2g) {
    case 0: rq_launch_one<F32, B, SS, 0>(grid, block, stream, p); break;
    case 1: rq_launch_one<F32, B, SS, 1>(grid, block, stream, p); break;
    case 2: rq_launch_one<F32, B, SS, 2>(grid, block, stream, p); break;
    case 3: rq_launch_one<F32, B, SS, 3>(grid, block, stream, p); break;
    case 4: rq_launch_one<F32, B, SS, 4>(grid, block, stream, p); break;
    case 5: rq_launch_one<F32, B, SS, 5>(grid, block, stream, p); break;
    case 6: rq_launch_one<F32, B, SS, 6>(grid, block, stream, p); break;
    case 7: rq_launch_one<F32, B, SS, 7>(grid, block, stream, p); break;
    default: rq_launch_one<F32, B, SS, 8>(grid, block, stream, p); break;
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
    if (sets == 1) rq_launch_one<F32, 4, 1, LG>(grid, block, stream, p);
    else if (sets == 2) rq_launch_one<F32, 4, 2, LG>(grid, block, stream, p);
    else rq_launch_one<F32, 4, 4, LG>(grid, block, stream, p);
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
    p.rinv = 1.0 / p.root;
    p.cg = (float)p.rinv;
    p.cg_lo = (float)(p.rinv - (double)p.cg);
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
