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
// Two kernels:
//  * unpack: packed nibbles -> int8 bytes 16*c (exact; low nibble (d << 4) & 0xF0F0F0F0, high
//    nibble d & 0xF0F0F0F0).  A packed dword's 8 codes come out as [c0 c2 c4 c6 | c1 c3 c5 c7]:
//    a fixed permutation inside every 8 channels, identical for tokens and weights, so every
//    dot product (and every 256-channel group) is unchanged.  The factor 16 * 16 = 256 is
//    removed with the scales;
//  * GEMM: the pipeline of the INT8 GEMM (persistent, XCD-aware tile order, 128-byte K-tiles
//    loaded global -> LDS with buffer_load ... lds, swizzled conflict-free fragment reads), with
//    3 LDS stages of 256 weight rows + 128 token rows.  8 wavefronts each own 64x64 outputs as
//    2x2 blocks of 32x32, with an int32 accumulator for the current group and an fp32 one for
//    the sum over groups (64 + 64 registers per lane).  A group is 2 K-tiles.  The group's
//    integer block is folded into the fp32 accumulator block by block inside the next group's
//    first MFMA sub-step, whose MFMAs start from a zero accumulator, so the fold's VALU work
//    overlaps the matrix pipe; the tile's last group is folded before its epilogue.  The
//    group's scales and the tile's bias are loaded into small LDS rings with the K-tiles.
#include "device_common.hpp"
#include "launchers.hpp"

namespace convrot {
namespace {

constexpr int BN = 256, BM = 128, BK = 128, NST = 3;
constexpr int WB = BN * BK, XB = BM * BK;         // bytes per stage: 32 KiB + 16 KiB
constexpr int STAGE = WB + XB;
constexpr int SC_OFF = NST * STAGE;               // 144 KiB
// One group's scales: sw as packed fp16 (512 B), then sx with one fp16 per dword (512 B).
constexpr int SC_BYTES = 2 * BN + 4 * BM;
constexpr int NSC = 4;                            // group-scale ring
constexpr int BIAS_OFF = SC_OFF + NSC * SC_BYTES;
constexpr int NBIAS = 4;                          // per-tile bias ring (fp32)
constexpr int SMEM = BIAS_OFF + NBIAS * BN * 4;
constexpr int NTHREADS = 512;
constexpr int GROUP_M = 8;
constexpr uint32_t OOB = 0x80000000u;
constexpr int NUM_RECORDS = 0x7ffffff0;

struct W4Params {
    const int8_t *xq;     // unpacked codes x16 [M, K]
    const int8_t *wq;     // unpacked codes x16 [N, K]
    const uint16_t *sx;   // [G, M] fp16
    const uint16_t *sw;   // [G, N] fp16
    const float *bias;
    void *y;
    int64_t M, N;
    int K;
    int tiles_m, tiles_n;
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }

__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__ushort_as_half(h); }

__device__ __forceinline__ void tile_of(int pid, int T, int tiles_m, int tiles_n, int &tm, int &tn)
{
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

// ---------------------------------------------------------------------------------------------
// unpack: 16 packed bytes (32 codes) per thread per step -> 32 int8 bytes

__global__ void __launch_bounds__(256) unpack_i4_kernel(const uint8_t *src, int8_t *dst, int64_t n16)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const v4u d = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(src) + i);
        v4u lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // packed dword e -> [lows | highs] = output dwords 2e, 2e+1
            const uint32_t l = (d[e] << 4) & 0xF0F0F0F0u, h = d[e] & 0xF0F0F0F0u;
            if (e < 2) { lo[2 * e] = l; lo[2 * e + 1] = h; }
            else { hi[2 * e - 4] = l; hi[2 * e - 3] = h; }
        }
        v4u *o = reinterpret_cast<v4u *>(dst) + 2 * i;
        o[0] = lo;
        o[1] = hi;
    }
}

// ---------------------------------------------------------------------------------------------

template <Epi E>
__global__ void __launch_bounds__(NTHREADS, 1) gemm_w4a4_kernel(W4Params p)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = w & 3, wm = w >> 2;         // wn: 64-row quarter of N, wm: 64-row half of M
    const int K = p.K;
    const int KT = K / BK;                     // even: K % 256 == 0
    const int G = K / 256;
    const int T = p.tiles_m * p.tiles_n;
    const int ntiles = (T - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int total = ntiles * KT;

    // Load geometry: weights, instruction i (0..3) of wave w fills rows 8*(8i+w) .. +7; tokens,
    // instruction i (0..1) fills rows 8*(8i+w) .. +7; lane -> row +lane/8, 16-byte position
    // lane%8 holding K chunk (lane%8) ^ swz(row).
    int lrow[4], lchunk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lrow[i] = 8 * (8 * i + w) + (lane >> 3);
        lchunk[i] = (lane & 7) ^ swz(lrow[i]);
    }

    int ld_t = -1, ld_tm = 0, ld_tn = 0;
    __amdgpu_buffer_rsrc_t rw, rx;
    uint32_t offw[4], offx[2];
    auto set_load_tile = [&](int t) {
        ld_t = t;
        tile_of((int)blockIdx.x + t * (int)gridDim.x, T, p.tiles_m, p.tiles_n, ld_tm, ld_tn);
        const int64_t m0 = (int64_t)ld_tm * BM, n0 = (int64_t)ld_tn * BN;
        rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(p.wq + n0 * K), (short)0, NUM_RECORDS, 0x00020000);
        rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(p.xq + m0 * K), (short)0, NUM_RECORDS, 0x00020000);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t o = (uint32_t)(lrow[i] * K + 16 * lchunk[i]);
            offw[i] = n0 + lrow[i] < p.N ? o : OOB;
            if (i < 2) offx[i] = m0 + lrow[i] < p.M ? o : OOB;
        }
    };
    // A group's scales go to ring slot (group & 3): waves 0 and 1 load the 256 sw values (4
    // bytes = 2 fp16 per lane; N % 8 == 0, so no dword straddles the end of the tile's rows);
    // waves 2 and 3 load the 128 sx values with 2-byte loads, which land zero-extended one per
    // dword, so a tile with an odd number of valid tokens still gets its last scale (a 4-byte
    // load half past the end would return 0).  A tile's bias (256 fp32) goes to ring slot
    // (tile & 3), loaded by waves 4..7.  Out-of-range entries and a missing bias read 0.
    auto issue_scales = [&](int gidx, int grp) {
        if constexpr (E == Epi::Bf16) {
            const int64_t m0 = (int64_t)ld_tm * BM, n0 = (int64_t)ld_tn * BN;
            const int64_t nrem = p.N - n0 < BN ? p.N - n0 : BN, mrem = p.M - m0 < BM ? p.M - m0 : BM;
            uint8_t *sb = smem + SC_OFF + (gidx & (NSC - 1)) * SC_BYTES;
            if (w < 2) {
                const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<uint16_t *>(p.sw + (int64_t)grp * p.N + n0), (short)0, (int)(2 * nrem), 0x00020000);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(sb + 256 * w), 4, (uint32_t)(256 * w + 4 * lane), 0, 0, 0);
            } else if (w < 4) {
                const int part = w - 2;
                const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<uint16_t *>(p.sx + (int64_t)grp * p.M + m0), (short)0, (int)(2 * mrem), 0x00020000);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(sb + 2 * BN + 256 * part), 2,
                                                         (uint32_t)(128 * part + 2 * lane), 0, 0, 0);
            }
        }
    };
    auto issue_bias = [&](int t) {
        if constexpr (E == Epi::Bf16) {
            if (w >= 4) {
                const int64_t n0 = (int64_t)ld_tn * BN;
                const int64_t nrem = p.N - n0 < BN ? p.N - n0 : BN;
                const int part = w - 4;
                // no bias: zero records, so every lane reads 0 without touching memory
                const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<float *>(p.bias ? p.bias + n0 : p.bias), (short)0, p.bias ? (int)(4 * nrem) : 0, 0x00020000);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)(smem + BIAS_OFF + (t & (NBIAS - 1)) * BN * 4 + 256 * part),
                                                         4, (uint32_t)(256 * part + 4 * lane), 0, 0, 0);
            }
        }
    };
    // Issue the next K-tile of the stream into stage (g % 3): 6 loads per wave, after the group
    // scales (even K-tiles) and the tile's bias (first K-tile).
    int ld_kt = 0, ld_g = 0;
    auto issue = [&](int g) {
        if (ld_kt == 0) {
            set_load_tile(ld_t + 1);
            issue_bias(ld_t);
        }
        if ((ld_kt & 1) == 0) issue_scales(ld_g++, ld_kt >> 1);
        const int k0 = __builtin_amdgcn_readfirstlane(ld_kt * BK);
        if (++ld_kt == KT) ld_kt = 0;
        uint8_t *base = smem + (g % NST) * STAGE + w * 1024;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(base + 8 * i * 1024), 16, offw[i], k0, 0, 0);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(base + WB + 8 * i * 1024), 16, offx[i], k0, 0, 0);
    };

    // Fragments: row = wave base + 32*blk + lane%32; sub-step kk (0..3) reads K chunk 2kk + lane/32.
    const int frow = lane & 31, fhalf = lane >> 5;
    const int arow = (wn * 64 + frow) * BK, brow = WB + (wm * 64 + frow) * BK;
    const int fpos[4] = {((0 + fhalf) ^ swz(frow)) * 16, ((2 + fhalf) ^ swz(frow)) * 16,
                         ((4 + fhalf) ^ swz(frow)) * 16, ((6 + fhalf) ^ swz(frow)) * 16};
    v4i fa[2][2], fb[2][2];
    auto read_frags = [&](int g, int kk, int buf) {
        const uint8_t *s0 = smem + (g % NST) * STAGE + fpos[kk];
#pragma unroll
        for (int b = 0; b < 2; ++b) fa[buf][b] = *reinterpret_cast<const v4i *>(s0 + arow + 32 * b * BK);
#pragma unroll
        for (int b = 0; b < 2; ++b) fb[buf][b] = *reinterpret_cast<const v4i *>(s0 + brow + 32 * b * BK);
    };
    v16i iacc[2][2];                         // current group (first written with a zero C)
    v16f facc[2][2];                         // sum over groups (zeroed at each tile's start)
    auto mfmas = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int bi = j >> 1, bj = j & 1;
            iacc[bi][bj] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[buf][bi], fb[buf][bj], iacc[bi][bj], 0, 0, 0);
        }
    };
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

    // Fold of block (bi, bj) of group with scale slot gidx into facc (zeroed at the tile's
    // start; a select between "first" and "accumulate" forms would cost the VALU both):
    // lane holds token m = lane%32 of the block and weight rows n = 8*(v/4) + 4*(lane/32) + v%4.
    // (16*16 = 256 is in sx / 256.)
    auto fold_block = [&](int gidx, int bi, int bj) {
        if constexpr (E == Epi::Int32) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int s = iacc[bi][bj][v] >> 8;       // exact: every product is 256 * cx * cw
                facc[bi][bj][v] = __int_as_float(__float_as_int(facc[bi][bj][v]) + s);
            }
        } else {
            const uint16_t *sb = reinterpret_cast<const uint16_t *>(smem + SC_OFF + (gidx & (NSC - 1)) * SC_BYTES);
            const uint32_t *sxd = reinterpret_cast<const uint32_t *>(sb + BN);          // one per dword
            const float sxm = f16_to_f32((uint16_t)sxd[wm * 64 + 32 * bj + frow]) * (1.0f / 256.0f);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = wn * 64 + 32 * bi + 8 * q + 4 * fhalf;
                const uint2 s2 = *reinterpret_cast<const uint2 *>(sb + nl);   // 4 fp16 scales
                const float sw4[4] = {f16_to_f32((uint16_t)(s2.x & 0xffff)), f16_to_f32((uint16_t)(s2.x >> 16)),
                                      f16_to_f32((uint16_t)(s2.y & 0xffff)), f16_to_f32((uint16_t)(s2.y >> 16))};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int v = 4 * q + e;
                    facc[bi][bj][v] = __builtin_fmaf((float)iacc[bi][bj][v], sxm * sw4[e], facc[bi][bj][v]);
                }
            }
        }
    };
    // First sub-step of a group: fold the previous group (if any) block by block, each right
    // before the zero-C MFMA that restarts that block.
    auto group_start = [&](bool fold, int gidx) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int bi = j >> 1, bj = j & 1;
            if (fold) fold_block(gidx, bi, bj);
            iacc[bi][bj] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[0][bi], fb[0][bj], v16i{}, 0, 0, 0);
            fence();
        }
    };

    // Epilogue of tile t: y = bf16(facc + bias), or the int32 total.  16-byte stores (N % 8 == 0).
    auto epilogue = [&](int t) {
        int tm, tn;
        tile_of((int)blockIdx.x + t * (int)gridDim.x, T, p.tiles_m, p.tiles_n, tm, tn);
        const int m0 = tm * BM, n0 = tn * BN;
        const int Mi = (int)p.M, Ni = (int)p.N;
        int erow = frow, ecol = wn * 64 + 4 * fhalf;
        asm volatile("" : "+v"(erow), "+v"(ecol));
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) {
            const int mr = m0 + wm * 64 + 32 * bj;
            const bool rok = mr + erow < Mi;
            if constexpr (E == Epi::Int32) {
                const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
                    static_cast<int32_t *>(p.y) + (int64_t)mr * p.N, (short)0, NUM_RECORDS, 0x00020000);
#pragma unroll
                for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int n = n0 + ecol + 32 * bi + 8 * g;
                        const v4u d = {__float_as_uint(facc[bi][bj][4 * g]), __float_as_uint(facc[bi][bj][4 * g + 1]),
                                       __float_as_uint(facc[bi][bj][4 * g + 2]), __float_as_uint(facc[bi][bj][4 * g + 3])};
                        const uint32_t off = (rok && n < Ni) ? (uint32_t)(erow * Ni + n) * 4u : OOB;
                        __builtin_amdgcn_raw_buffer_store_b128(d, ry, off, 0, 0);
                    }
            } else {
                const float *lb = reinterpret_cast<const float *>(smem + BIAS_OFF + (t & (NBIAS - 1)) * BN * 4);
                const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
                    static_cast<uint16_t *>(p.y) + (int64_t)mr * p.N, (short)0, NUM_RECORDS, 0x00020000);
#pragma unroll
                for (int bi = 0; bi < 2; ++bi)
#pragma unroll
                    for (int g2 = 0; g2 < 2; ++g2) {
                        uint32_t pk[2][2];
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int g = 2 * g2 + h;
                            const v4f b4 = *reinterpret_cast<const v4f *>(lb + ecol + 32 * bi + 8 * g);
                            pk[h][0] = pack_bf16x2(facc[bi][bj][4 * g] + b4[0], facc[bi][bj][4 * g + 1] + b4[1]);
                            pk[h][1] = pack_bf16x2(facc[bi][bj][4 * g + 2] + b4[2], facc[bi][bj][4 * g + 3] + b4[3]);
                        }
                        // lane l < 32 takes columns 8g..8g+7 of group 2*g2, lane l+32 of 2*g2+1
                        swap32(pk[0][0], pk[1][0]);
                        swap32(pk[0][1], pk[1][1]);
                        const int n = n0 + (ecol - 4 * fhalf) + 32 * bi + 8 * (2 * g2 + fhalf);
                        const uint32_t off = (rok && n < Ni) ? (uint32_t)(erow * Ni + n) * 2u : OOB;
                        __builtin_amdgcn_raw_buffer_store_b128(v4u{pk[0][0], pk[0][1], pk[1][0], pk[1][1]}, ry, off, 0, 0);
                    }
            }
        }
    };

    if (ntiles <= 0) return;
    constexpr int LPW = 6;                                  // K-tile loads per wave
    constexpr int EPI_STORES = E == Epi::Int32 ? 16 : 8;   // stores per wave after an epilogue
    issue(0);
    if (total > 1) issue(1);
    if (total > 2) issue(2);
    if (total > 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * LPW));
    else if (total > 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPW));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    read_frags(0, 0, 0);

    int g = 0, gidx = 0;                                    // gidx: this stream's group index
    for (int t = 0; t < ntiles; ++t) {
        for (int kt = 0; kt < KT; ++kt, ++g) {
            if ((kt & 1) == 0) {
                // first K-tile of a group: restart the int32 blocks (folding the previous group)
                if (kt == 0) {
#pragma unroll
                    for (int a = 0; a < 2; ++a)
#pragma unroll
                        for (int b = 0; b < 2; ++b) facc[a][b] = v16f{};
                }
                group_start(kt > 0, gidx - 1);
                fence();
                read_frags(g, 1, 1);
            } else {
                read_frags(g, 1, 1);
                fence();
                mfmas(0);
            }
            fence();
            read_frags(g, 2, 0);
            fence();
            mfmas(1);
            fence();
            read_frags(g, 3, 1);
            fence();
            mfmas(0);
            fence();
            // K-tile g+1 must have landed: at most K-tile g+2's loads (and, in a tile's first
            // two K-tiles, the previous tile's epilogue stores) may still be in flight.
            if (g + 2 < total) {
                if (t > 0 && kt < 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPW + EPI_STORES));
                else __builtin_amdgcn_s_waitcnt(waitcnt_vm(LPW));
            } else {
                __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            }
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            if (g + 3 < total) issue(g + 3);
            if (g + 1 < total) read_frags(g + 1, 0, 0);
            fence();
            mfmas(1);
            fence();
            if (kt & 1) ++gidx;
        }
        // the tile's last group, then its epilogue
#pragma unroll
        for (int j = 0; j < 4; ++j) fold_block(gidx - 1, j >> 1, j & 1);
        epilogue(t);
    }
}

int cu_count()
{
    static int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            n = 256;
        return n > 0 ? n : 256;
    }();
    return cus;
}

} // namespace

size_t w4a4_unpacked_bytes(int64_t M, int64_t N, int K) { return (size_t)(M + N) * (size_t)K; }

hipError_t launch_gemm_w4a4(const uint8_t *xq, const uint8_t *wq, const uint16_t *sx, const uint16_t *sw,
                            const float *bias, void *y, Epi epi, int64_t M, int64_t N, int K, void *ws,
                            hipStream_t stream)
{
    if (M <= 0 || N <= 0) return hipSuccess;
    int8_t *xu = static_cast<int8_t *>(ws);
    int8_t *wu = xu + M * (int64_t)K;
    // unpack both operands (K/32 16-byte blocks per row)
    const int64_t nx = M * (K / 32), nw = N * (K / 32);
    const unsigned ugrid = (unsigned)(cu_count() * 8);
    hipLaunchKernelGGL(unpack_i4_kernel, dim3(ugrid), dim3(256), 0, stream, xq, xu, nx);
    hipLaunchKernelGGL(unpack_i4_kernel, dim3(ugrid), dim3(256), 0, stream, wq, wu, nw);
    W4Params p;
    p.xq = xu;
    p.wq = wu;
    p.sx = sx;
    p.sw = sw;
    p.bias = bias;
    p.y = y;
    p.M = M;
    p.N = N;
    p.K = K;
    p.tiles_m = (int)((M + BM - 1) / BM);
    p.tiles_n = (int)((N + BN - 1) / BN);
    const int T = p.tiles_m * p.tiles_n;
    int grid = cu_count();
    if (T < grid) grid = (T + 7) & ~7;
    if (epi == Epi::Int32)
        hipLaunchKernelGGL(gemm_w4a4_kernel<Epi::Int32>, dim3((unsigned)grid), dim3(NTHREADS), 0, stream, p);
    else
        hipLaunchKernelGGL(gemm_w4a4_kernel<Epi::Bf16>, dim3((unsigned)grid), dim3(NTHREADS), 0, stream, p);
    return hipGetLastError();
}

} // namespace convrot
