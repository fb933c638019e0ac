// gemm_w4a4.hip -- W4A4 ConvRot linear on the INT8 MFMA core (gfx950).
//
// Both operands were rotated by the grouped Hadamard and quantized to 4-bit codes with one fp16
// scale per (row, 256-channel group) ("minimax-h3-nvfp4-convrot核心原理", section 五: W4A4 rotates
// activations and weights and quantizes to 4 bits, RTN).  gfx950 has no INT4 matrix instruction,
// so the codes are widened to INT8 and run through v_mfma_i32_32x32x32_i8:
//   y[m,n] = sum_g ( sum_{k in g} cx[m,k] cw[n,k] ) * sx[g,m] * sw[g,n] + bias[n]
// Each group's integer dot products are exact; they are scaled and summed in fp32 in
// increasing group order.
//
// Design:
//  * workgroup tile 256 (weight rows) x 128 (tokens); 4 wavefronts in 2x2, each 128x64 =
//    4x2 blocks of 32x32 (128 int32 + 128 fp32 accumulators per lane);
//  * a stage is 128 codes (64 packed bytes) per row.  Packed tiles are loaded into registers one
//    stage ahead and widened once per workgroup while being written to LDS: a nibble c becomes
//    the byte 16*c (low nibbles: (d << 4) & 0xF0F0F0F0, high nibbles: d & 0xF0F0F0F0), which is
//    exact in int8; the factor 16*16 = 256 is removed with the scale.  Weight and token rows get
//    the identical byte permutation, so the K order inside a stage is consistent for the MFMA;
//  * after every second stage (one group) the integer block is folded into the fp32
//    accumulators with that group's scales, which are prefetched from global memory at the
//    start of the group (scales are stored group-major, [K/256, rows], so a group is contiguous).
#include "device_common.hpp"
#include "launchers.hpp"

namespace convrot {
namespace {

constexpr int BN = 256, BM = 128;
constexpr int BKC = 128;                      // codes (= unpacked bytes) per row per stage
constexpr int WB = BN * BKC, XB = BM * BKC;   // unpacked bytes per stage
constexpr int STAGE = WB + XB;                // 48 KiB
constexpr int EPI_PITCH = BN * 2 + 16;
constexpr int SMEM = (2 * STAGE > BM * EPI_PITCH) ? 2 * STAGE : BM * EPI_PITCH;
constexpr int GROUP_M = 8;

struct W4Params {
    const uint8_t *xq;
    const uint8_t *wq;
    const uint16_t *sx;   // [G, M] fp16
    const uint16_t *sw;   // [G, N] fp16
    const float *bias;
    void *y;
    int64_t M, N;
    int K;
    int tiles_m, tiles_n;
};

__device__ __forceinline__ void tile_of(int pid, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int T = tiles_m * tiles_n;
    const int xcd = pid & 7, local = pid >> 3;
    const int per = T >> 3, rem = T & 7;
    const int q = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
    const int span = GROUP_M * tiles_n;
    const int first_m = (q / span) * GROUP_M;
    const int gsz = min(tiles_m - first_m, GROUP_M);
    const int r = q % span;
    tm = first_m + r % gsz;
    tn = r / gsz;
}

__device__ __forceinline__ float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

template <Epi E>
__global__ void __launch_bounds__(256, 1) gemm_w4a4_kernel(W4Params p)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int wn = w & 1, wm = w >> 1;
    int tm, tn;
    tile_of(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int Kb = p.K / 2;                 // packed bytes per row
    const int ST = p.K / BKC;               // stages (2 per group)

    // Global packed chunks (16 bytes = 32 codes) this thread loads per stage: 4 weight chunks
    // (rows t/4 + 64i, chunk t%4) and 2 token chunks (rows t/4 + 64i).
    const int crow = t >> 2, cch = t & 3;
    const uint8_t *gw[4];
    const uint8_t *gx[2];
    bool okx[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int64_t n = n0 + crow + 64 * i;
        n = n < p.N ? n : p.N - 1;          // rows >= N are computed but never stored
        gw[i] = p.wq + n * Kb + 16 * cch;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t m = m0 + crow + 64 * i;
        okx[i] = m < p.M;
        gx[i] = p.xq + (okx[i] ? m : 0) * Kb + 16 * cch;
    }
    v4u pw[4], px[2];
    auto gload = [&](int st) {
        const int off = st * (BKC / 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) pw[i] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(gw[i] + off));
#pragma unroll
        for (int i = 0; i < 2; ++i) px[i] = okx[i] ? *reinterpret_cast<const v4u *>(gx[i] + off) : v4u{0u, 0u, 0u, 0u};
    };
    // Packed chunk c of a row -> unpacked chunks 2c (low nibbles) and 2c+1 (high nibbles),
    // stored at swizzled 16-byte positions u ^ (row & 7).
    auto widen_store = [&](int buf) {
        uint8_t *s0 = smem + buf * STAGE;
        auto put = [&](uint8_t *base, int row, v4u d) {
            const uint4 lo = make_uint4((d.x << 4) & 0xf0f0f0f0u, (d.y << 4) & 0xf0f0f0f0u, (d.z << 4) & 0xf0f0f0f0u,
                                        (d.w << 4) & 0xf0f0f0f0u);
            const uint4 hi = make_uint4(d.x & 0xf0f0f0f0u, d.y & 0xf0f0f0f0u, d.z & 0xf0f0f0f0u, d.w & 0xf0f0f0f0u);
            const int sw = row & 7;
            *reinterpret_cast<uint4 *>(base + row * BKC + 16 * ((2 * cch) ^ sw)) = lo;
            *reinterpret_cast<uint4 *>(base + row * BKC + 16 * ((2 * cch + 1) ^ sw)) = hi;
        };
#pragma unroll
        for (int i = 0; i < 4; ++i) put(s0, crow + 64 * i, pw[i]);
#pragma unroll
        for (int i = 0; i < 2; ++i) put(s0 + WB, crow + 64 * i, px[i]);
    };

    v16i iacc[4][2];
    v16f facc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            iacc[a][b] = v16i{};
            facc[a][b] = v16f{};
        }

    const int frow = lane & 31, fhalf = lane >> 5, fsw = lane & 7;
    // scales of the current group for this lane's rows: tokens m (one per bj), weight rows n
    // (4 consecutive per (bi, quarter))
    uint16_t rsx[2];
    uint2 rsw[4][4];
    auto load_scales = [&](int g) {
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
            int64_t m = m0 + wm * 64 + 32 * bj + frow;
            m = m < p.M ? m : p.M - 1;
            rsx[bj] = p.sx[(int64_t)g * p.M + m];
        }
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                int64_t n = n0 + wn * 128 + 32 * bi + 8 * qq + 4 * fhalf;
                n = n < p.N ? n : p.N - 4;
                rsw[bi][qq] = *reinterpret_cast<const uint2 *>(p.sw + (int64_t)g * p.N + n);
            }
    };

    gload(0);
    widen_store(0);
    __syncthreads();
    for (int st = 0; st < ST; ++st) {
        const int buf = st & 1;
        if (st + 1 < ST) gload(st + 1);
        if constexpr (E == Epi::Bf16) {
            if (!(st & 1)) load_scales(st >> 1);
        }
        const uint8_t *sa = smem + buf * STAGE;
        const uint8_t *sb = sa + WB;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int pos = ((2 * kk + fhalf) ^ fsw) * 16;
            v4i fa[4], fb[2];
#pragma unroll
            for (int bi = 0; bi < 4; ++bi) fa[bi] = *reinterpret_cast<const v4i *>(sa + (wn * 128 + 32 * bi + frow) * BKC + pos);
#pragma unroll
            for (int bj = 0; bj < 2; ++bj) fb[bj] = *reinterpret_cast<const v4i *>(sb + (wm * 64 + 32 * bj + frow) * BKC + pos);
#pragma unroll
            for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                for (int bj = 0; bj < 2; ++bj)
                    iacc[bi][bj] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[bi], fb[bj], iacc[bi][bj], 0, 0, 0);
        }
        if constexpr (E == Epi::Bf16) {
            if (st & 1) {
                // fold this group into fp32: 32x32 block layout, lane holds token m = lane%32 and
                // weight rows n = 8*(v/4) + 4*(lane/32) + v%4.  1/256 undoes the 16x16 widening.
#pragma unroll
                for (int bj = 0; bj < 2; ++bj) {
                    const float sxv = h2f(rsx[bj]) * (1.0f / 256.0f);
#pragma unroll
                    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                        for (int qq = 0; qq < 4; ++qq) {
                            const uint2 s4 = rsw[bi][qq];
                            const float sv[4] = {h2f((uint16_t)(s4.x & 0xffff)), h2f((uint16_t)(s4.x >> 16)),
                                                 h2f((uint16_t)(s4.y & 0xffff)), h2f((uint16_t)(s4.y >> 16))};
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                facc[bi][bj][4 * qq + i] =
                                    __builtin_fmaf((float)iacc[bi][bj][4 * qq + i], sxv * sv[i], facc[bi][bj][4 * qq + i]);
                        }
                }
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b) iacc[a][b] = v16i{};
            }
        }
        if (st + 1 < ST) {
            __syncthreads();            // everyone is done reading the buffer about to be refilled
            widen_store(buf ^ 1);
        }
        __syncthreads();
    }

    if constexpr (E == Epi::Int32) {
        int32_t *y = static_cast<int32_t *>(p.y);
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
            const int64_t m = m0 + wm * 64 + 32 * bj + frow;
            if (m >= p.M) continue;
#pragma unroll
            for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t n = n0 + wn * 128 + 32 * bi + 8 * (v >> 2) + 4 * fhalf + (v & 3);
                    if (n < p.N) y[m * p.N + n] = iacc[bi][bj][v] >> 8;   // exact: every product carries 16*16
                }
        }
    } else {
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
            const int ml = wm * 64 + 32 * bj + frow;
#pragma unroll
            for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int nl = wn * 128 + 32 * bi + 8 * qq + 4 * fhalf;
                    float yv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t n = n0 + nl + i;
                        yv[i] = facc[bi][bj][4 * qq + i] + ((p.bias && n < p.N) ? p.bias[n] : 0.0f);
                    }
                    uint2 pk;
                    pk.x = pack_bf16x2(yv[0], yv[1]);
                    pk.y = pack_bf16x2(yv[2], yv[3]);
                    *reinterpret_cast<uint2 *>(smem + ml * EPI_PITCH + nl * 2) = pk;
                }
        }
        __syncthreads();
        uint16_t *y = static_cast<uint16_t *>(p.y);
        const int ch = t & 31;
        for (int rp = 0; rp < BM; rp += 8) {
            const int row = rp + (t >> 5);
            const int64_t m = m0 + row, n = n0 + 8 * ch;
            if (m >= p.M || n >= p.N) continue;
            *reinterpret_cast<uint4 *>(y + m * p.N + n) = *reinterpret_cast<const uint4 *>(smem + row * EPI_PITCH + 16 * ch);
        }
    }
}

} // namespace

hipError_t launch_gemm_w4a4(const uint8_t *xq, const uint8_t *wq, const uint16_t *sx, const uint16_t *sw,
                            const float *bias, void *y, Epi epi, int64_t M, int64_t N, int K, hipStream_t stream)
{
    if (M <= 0 || N <= 0) return hipSuccess;
    W4Params p;
    p.xq = xq;
    p.wq = wq;
    p.sx = sx;
    p.sw = sw;
    p.bias = bias;
    p.y = y;
    p.M = M;
    p.N = N;
    p.K = K;
    p.tiles_m = (int)((M + BM - 1) / BM);
    p.tiles_n = (int)((N + BN - 1) / BN);
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(256);
    if (epi == Epi::Int32)
        hipLaunchKernelGGL(gemm_w4a4_kernel<Epi::Int32>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(gemm_w4a4_kernel<Epi::Bf16>, grid, block, 0, stream, p);
    return hipGetLastError();
}

} // namespace convrot
