// gemm_w4a4.hip -- W4A4 ConvRot linear on the FP6 matrix instructions of gfx950.
//
// Both operands were rotated by the grouped Hadamard and quantized to 4-bit codes with one fp16
// scale per (row, 256-channel group) ("minimax-h3-nvfp4-convrot核心原理", section 五: W4A4 rotates
// activations and weights and quantizes to 4 bits, RTN):
//   y[m,n] = sum_g ( sum_{k in g} cx[m,k] cw[n,k] ) * sx[g,m] * sw[g,n] + bias[n]
// gfx950 has no INT4 matrix instruction, but every 4-bit code (-8..7) is exactly an FP6 E3M2
// value (OCP MX: sign, 3 exponent bits with bias 3, 2 mantissa bits), and
// v_mfma_scale_f32_32x32x64_f8f6f4 multiplies FP6 operands at twice the INT8 rate with fp32
// accumulation.  A group's 256 products are integers of magnitude <= 64 * 256, so its fp32 sum
// is exact: the same integer the INT8 core would give.  The block-scale operands stay at 2^0;
// the fp16 scales are applied afterwards in fp32, group by group in increasing order.
//
// Two kernels:
//  * tile: packed nibbles -> FP6 in the order the MFMA consumes them (weights once, or tokens
//    given as packed codes).  Per 32-row block and
//    64-channel K-step one 1536-byte piece; lane l = (r = l % 32, h = l / 32) owns the 32 codes
//    of row r at channels 64 ks + 32 h + s (s = 0..31), 6 bits each at bit 6 s of a 24-byte
//    string whose first 16 bytes sit at 16 l and last 8 at 1024 + 8 l.  Pieces are ordered
//    [row block][K-step], so a row block's two K-steps of a 128-channel K-tile are 3 KiB of
//    contiguous memory that 16-byte loads-to-LDS copy verbatim, and a fragment is one 16-byte
//    and one 8-byte LDS read, both conflict-free.  Rows past the operand's end are zeros;
//  * GEMM: persistent, XCD-aware tile order, 256 weight rows x 128 token rows per workgroup,
//    K-tiles of 128 channels (3 KiB per row block) loaded global -> LDS with buffer_load ... lds
//    into NST stages.  8 wavefronts each own 64x64 outputs as 2x2 blocks of 32x32, with an fp32
//    accumulator for the current 256-group and one for the sum over groups (64 + 64 registers
//    per lane).  A group's block is folded into the sum right before the next group's first
//    MFMA restarts it from zero; the scale product sx[m] * sw[n] of a block comes from one
//    f16 MFMA (an outer product), so the fold costs one FMA per output.  The tile's last group
//    is folded before its epilogue.  The group's scales and the tile's bias ride in small LDS
//    rings with the K-tiles.
//
// Built with machine sinking off (-mllvm -disable-machine-sink): otherwise the fold's FMAs and
// MFMAs are sunk past the load-issue branches into the next block, after the barrier, where
// they no longer overlap the matrix pipe and the register pressure spills.
#include "device_common.hpp"
#include "launchers.hpp"

namespace convrot {
namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

constexpr int PIECE = 1536;                       // one 32-row block x 64 channels of FP6
constexpr int CHUNK = 2 * PIECE;                  // one 32-row block x one 128-channel K-tile
constexpr int BN = 256, BM = 128, BK = 128, NST = 4;
constexpr int WB = (BN / 32) * CHUNK, XB = (BM / 32) * CHUNK;   // 24 KiB + 12 KiB per stage
constexpr int STAGE = WB + XB;
constexpr int DUMMY_OFF = NST * STAGE;            // 1 KiB target of the padding loads
constexpr int SC_OFF = DUMMY_OFF + 1024;
// One group's scales: sw as packed fp16 (512 B), then sx with one fp16 per dword (512 B).
constexpr int SC_BYTES = 2 * BN + 4 * BM;
constexpr int NSC = 8;                            // group-scale ring (>= NST + 2 groups of one K-tile)
constexpr int BIAS_OFF = SC_OFF + NSC * SC_BYTES;
constexpr int NBIAS = 4;                          // per-tile bias ring (fp32)
constexpr int ZERO_OFF = BIAS_OFF + NBIAS * BN * 4; // 16 zero bytes
constexpr int SMEM = ZERO_OFF + 16;
static_assert(SMEM <= 160 * 1024, "LDS budget");
constexpr int NTHREADS = 512;
constexpr int GROUP_M = 8;
constexpr uint32_t OOB = 0x80000000u;
constexpr int NUM_RECORDS = 0x7ffffff0;


struct W4Params {
    const uint8_t *xt;    // tokens, FP6 tiles [ceil(M/32)][K/64][1536]
    const uint8_t *wt;    // weights, FP6 tiles [ceil(N/32)][K/64][1536]
    const uint16_t *sx;   // [G, M] fp16
    const uint16_t *sw;   // [G, N] fp16
    const float *bias;
    void *y;
    int64_t M, N;
    int K;
    int tiles_m, tiles_n;
};

typedef __attribute__((address_space(3))) void lds_void;

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

__device__ __forceinline__ v16f mfma_fp6(const v8i &a, const v8i &b, const v16f &c)
{
    // cbsz = blgp = 3: both operands FP6 E3M2; scale operands 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 3, 3, 0, 127, 0, 127);
}

// ---------------------------------------------------------------------------------------------
// tile: a workgroup re-encodes 32 rows x 256 channels (4 pieces) per unit.  Thread t reads the
// 16 packed bytes (32 codes) of row t/8 at channel chunk t%8, so a wavefront reads 8 whole
// 128-byte lines, and those 32 codes are exactly what lane (row, chunk%2) of piece (chunk/2)
// holds: 24 bytes out.  The codes become integer-valued floats (sign-extending bit-field
// extracts) and one v_cvt_scalef32_2xpk16_bf6_f32 packs them as E3M2 (output position 2i + b
// from element i of source b: the even channels, i.e. the low nibbles, are source 0; scale 1,
// exact for integers up to 8 in magnitude).  A thread takes TILE_U units per iteration with all
// their loads in flight first.  Out-of-range rows and channels lie past num_records: they read
// zeros and their stores drop.  K % 128 == 0: with K % 256 == 128 a row block's last unit has
// only 2 pieces.

constexpr int TILE_U = 2;

__global__ void __launch_bounds__(256) tile_fp6_kernel(const uint8_t *src, uint8_t *dst, int64_t R, int K,
                                                       uint32_t units)
{
    const uint32_t KS = (uint32_t)K >> 6, KQ = ((uint32_t)K + 255) >> 8;
    const uint32_t r = threadIdx.x >> 3, c = threadIdx.x & 7;
    const uint32_t l = r + 32 * (c & 1);                     // lane of the piece
    for (uint32_t u0 = blockIdx.x; u0 < units; u0 += TILE_U * gridDim.x) {
        v4u d[TILE_U];
#pragma unroll
        for (int i = 0; i < TILE_U; ++i) {
            const uint32_t u = u0 + i * gridDim.x;
            const uint32_t rb = u / KQ, q = u - rb * KQ;
            const int64_t row0 = 32 * (int64_t)rb;
            const int64_t nrows = R - row0 < 32 ? R - row0 : 32;
            const bool ok = u < units && 4 * q + (c >> 1) < KS;
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t *>(src) + (ok ? row0 * (K >> 1) : 0), (short)0,
                ok && nrows > 0 ? (int)(nrows * (K >> 1)) : 0, 0x00020000);
            d[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? r * (uint32_t)(K >> 1) + 128 * q + 16 * c : OOB, 0, 2);
        }
#pragma unroll
        for (int i = 0; i < TILE_U; ++i) {
            const uint32_t u = u0 + i * gridDim.x;
            const uint32_t rb = u / KQ, q = u - rb * KQ;
            const uint32_t ks = 4 * q + (c >> 1);                // K-step of this thread's piece
            if (u >= units || ks >= KS) continue;
            v16f f[2];
#pragma unroll
            for (int b = 0; b < 16; ++b) {
                const uint32_t w = d[i][b >> 2];
                f[0][b] = (float)(int)__builtin_amdgcn_sbfe((int)w, 8 * (b & 3), 4);
                f[1][b] = (float)(int)__builtin_amdgcn_sbfe((int)w, 8 * (b & 3) + 4, 4);
            }
            typedef unsigned v6u __attribute__((ext_vector_type(6)));
            const v6u o = __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(f[0], f[1], 1.0f);
            uint8_t *piece = dst + ((int64_t)rb * KS + ks) * PIECE;
            *reinterpret_cast<v4u *>(piece + 16 * l) = v4u{o[0], o[1], o[2], o[3]};
            *reinterpret_cast<v2u *>(piece + 1024 + 8 * l) = v2u{o[4], o[5]};
        }
    }
}

// ---------------------------------------------------------------------------------------------

// GKT: K-tiles per scale group (2 for 256-channel groups, 1 for 128-channel ones).
template <Epi E, int GKT>
__global__ void __launch_bounds__(NTHREADS, 1) gemm_w4a4_kernel(W4Params p)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = w & 3, wm = w >> 2;         // wn: 64-row quarter of N, wm: 64-row half of M
    const int K = p.K;
    const int KT = K / BK;                     // a multiple of GKT
    const int G = KT / GKT;
    const int KSTRIDE = (K / 64) * PIECE;      // bytes between consecutive row blocks
    const int T = p.tiles_m * p.tiles_n;
    const int ntiles = (T - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int total = ntiles * KT;
    const int nblk_w = (int)((p.N + 31) >> 5), nblk_x = (int)((p.M + 31) >> 5);

    // Load geometry: a K-tile is 24 weight and 12 token 1 KiB pieces; wave w issues weight
    // pieces w, w + 8, w + 16 and token pieces w and w + 8 (waves 4..7: a padding load to the
    // 1 KiB dummy area instead, so every wave issues the same number of loads).  Piece d of a
    // row-block chunk array is row block d / 3, third d % 3, and lands at LDS offset 1024 d.
    int ld_t = -1, ld_tm = 0, ld_tn = 0;
    __amdgpu_buffer_rsrc_t rw, rx;
    // Per load: the lane's 16-byte position as voffset (with bit 31 set when the row block lies
    // past the operand, so the load returns zeros without touching memory) and the wave-uniform
    // rest (row block and third) in soffset.
    const uint32_t lane16 = 16u * (uint32_t)lane;
    uint32_t sow[3], sox[2], oobw[3], oobx[2];
    auto set_load_tile = [&](int t) {
        ld_t = t;
        tile_of((int)blockIdx.x + t * (int)gridDim.x, T, p.tiles_m, p.tiles_n, ld_tm, ld_tn);
        const int bw0 = ld_tn * (BN / 32), bx0 = ld_tm * (BM / 32);
        rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.wt + (int64_t)bw0 * KSTRIDE), (short)0,
                                               NUM_RECORDS, 0x00020000);
        rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.xt + (int64_t)bx0 * KSTRIDE), (short)0,
                                               NUM_RECORDS, 0x00020000);
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int d = w + 8 * i, j = d / 3;
            sow[i] = (uint32_t)(j * KSTRIDE + 1024 * (d % 3));
            oobw[i] = bw0 + j < nblk_w ? 0u : OOB;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int d = w + 8 * i, j = d / 3;
            sox[i] = d < 12 ? (uint32_t)(j * KSTRIDE + 1024 * (d % 3)) : 0u;
            oobx[i] = d < 12 && bx0 + j < nblk_x ? 0u : OOB;
        }
    };
    // A group's scales go to ring slot (group & 7): waves 0 and 1 load the 256 sw values (4
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
    // Issue the next K-tile of the stream into stage (g % NST): 5 loads per wave, after the
    // group scales (a group's first K-tile) and the tile's bias (first K-tile).
    int ld_kt = 0, ld_g = 0;
    auto issue = [&](int g) {
        if (ld_kt == 0) {
            set_load_tile(ld_t + 1);
            issue_bias(ld_t);
        }
        if (ld_kt % GKT == 0) issue_scales(ld_g++, ld_kt / GKT);
        const int k0 = __builtin_amdgcn_readfirstlane(ld_kt * CHUNK);
        if (++ld_kt == KT) ld_kt = 0;
        uint8_t *base = smem + (g % NST) * STAGE;
#pragma unroll
        for (int i = 0; i < 3; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(base + 1024 * (w + 8 * i)), 16, lane16 | oobw[i],
                                                     k0 + sow[i], 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(base + WB + 1024 * w), 16, lane16 | oobx[0], k0 + sox[0],
                                                 0, 0);
        // waves 4..7: token piece w + 8 does not exist; the load is out of range and the zeros
        // land in the dummy area
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rx, (lds_void *)(w < 4 ? base + WB + 1024 * (w + 8) : smem + DUMMY_OFF), 16, lane16 | oobx[1], k0 + sox[1],
            0, 0);
    };

    // Fragments: weight block bi of the wave is row block 2 wn + bi, token block bj is row block
    // 2 wm + bj; K-step ks of the K-tile is the piece at ks * 1536 inside the block's chunk.  A
    // lane's 24 bytes are one 16-byte read (bytes 0..1023 of the piece) and one 8-byte read
    // (bytes 1024..1535), which land in the operand's 6 consecutive registers.  Each fragment
    // gets its own address register for the 8-byte read: with a shared one the compiler pairs
    // the reads of two fragments into one ds_read2 and must then copy the halves apart.
    const int frow = lane & 31, fhalf = lane >> 5;
    const int lane8 = 1024 + 8 * lane;
    v8i fa[2][2], fb[2][2];
    auto join = [](const v4i &a, const v2i &b) {
        const v4i bb = __builtin_shufflevector(b, b, 0, 1, -1, -1);
        return __builtin_shufflevector(a, bb, 0, 1, 2, 3, 4, 5, -1, -1);
    };
    auto read_frags = [&](int g, int ks, int buf) {
        const int so = (g % NST) * STAGE + ks * PIECE;
        const uint8_t *h = smem + so + lane16;
        int t[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            // f = 0, 1: weight blocks; 2, 3: token blocks
            t[f] = lane8 + so + (f < 2 ? (2 * wn + f) * CHUNK : WB + (2 * wm + f - 2) * CHUNK);
            asm volatile("" : "+v"(t[f]));
        }
#pragma unroll
        for (int b = 0; b < 2; ++b)
            fa[buf][b] = join(*reinterpret_cast<const v4i *>(h + (2 * wn + b) * CHUNK),
                              *reinterpret_cast<const v2i *>(smem + t[b]));
#pragma unroll
        for (int b = 0; b < 2; ++b)
            fb[buf][b] = join(*reinterpret_cast<const v4i *>(h + WB + (2 * wm + b) * CHUNK),
                              *reinterpret_cast<const v2i *>(smem + t[2 + b]));
    };
    v16f gacc[2][2];                         // current group (first written with a zero C)
    v16f facc[2][2];                         // sum over groups (zeroed at each tile's start)
    auto mfmas = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int bi = j >> 1, bj = j & 1;
            gacc[bi][bj] = mfma_fp6(fa[buf][bi], fb[buf][bj], gacc[bi][bj]);
        }
    };
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    // Inside one scheduling region, the next K-step's fragment reads go out two at a time between
    // this K-step's MFMAs (sched_group_barrier masks: 0x008 MFMA, 0x100 LDS read), so the matrix
    // pipe gets its next instruction without queueing behind a burst of reads.
    auto interleave_reads = [] {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
    };

    // Fold of a group into facc (zeroed at the tile's start): facc += gacc * sx[m] * sw[n].
    // Lane holds token m = lane%32 of block (bi, bj) and weight rows n = 8*(v/4) + 4*(lane/32) + v%4.
    // The per-output scale product P = sw[n] * sx[m] of each 32x32 block is an outer product,
    // made by one f16 MFMA with K = 8 of which only k = 0 is non-zero: A row i holds sw of the
    // block's weight row i, B column j holds sx of its token j, so P lands in the accumulator's
    // own layout, exact (a product of two fp16 values fits fp32).  The fold is then one FMA per
    // output, the same fma(acc, sx*sw, facc) as an exact-product reference.  A lane < 32 loads
    // its k = 0 entry zero-extended (k = 1..3 zero); lanes >= 32 (k = 4..7) read, for A, the
    // finite scale of lane - 32 and, for B, the zero slot, so every k >= 1 term is 0.
    v4h pa[2], pb[2];
    auto read_scales = [&](int gidx) {
        // offsets formed here from the lane id (short-lived registers)
        int l = lane;
        asm volatile("" : "+v"(l));
        const int sw_off = 2 * (wn * 64 + (l & 31));                                 // + 64 * bi
        const int sx_off = l < 32 ? 2 * BN + 4 * (wm * 64 + (l & 31)) : -1;          // + 128 * bj
        const uint8_t *sb = smem + SC_OFF + (gidx & (NSC - 1)) * SC_BYTES;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint32_t a = *reinterpret_cast<const uint16_t *>(sb + sw_off + 64 * b);
            pa[b] = __builtin_bit_cast(v4h, v2u{a, 0u});
            const uint32_t x = *reinterpret_cast<const uint32_t *>(
                sx_off >= 0 ? sb + sx_off + 128 * b : smem + ZERO_OFF);
            pb[b] = __builtin_bit_cast(v4h, v2u{x, 0u});
        }
    };
    auto fold_block = [&](int bi, int bj) {
        if constexpr (E == Epi::Int32) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int s = (int)gacc[bi][bj][v];       // exact: an integer below 2^24
                facc[bi][bj][v] = __int_as_float(__float_as_int(facc[bi][bj][v]) + s);
            }
        } else {
            // keep each block's scale product next to its fold (hoisting all four would hold
            // 64 more registers)
            v4h a = pa[bi];
            asm volatile("" : "+v"(a));
            const v16f pr = __builtin_amdgcn_mfma_f32_32x32x8f16(a, pb[bj], v16f{}, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 16; ++v) facc[bi][bj][v] = __builtin_fmaf(gacc[bi][bj][v], pr[v], facc[bi][bj][v]);
        }
    };
    // First K-step of a group: fold the previous group (if any) block by block, each right
    // before the zero-C MFMA that restarts that block.
    auto group_start = [&](bool fold, int gidx) {
        if (fold && E == Epi::Bf16) read_scales(gidx);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int bi = j >> 1, bj = j & 1;
            if (fold) fold_block(bi, bj);
            gacc[bi][bj] = mfma_fp6(fa[0][bi], fb[0][bj], v16f{});
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
    if (threadIdx.x < 4) reinterpret_cast<uint32_t *>(smem + ZERO_OFF)[threadIdx.x] = 0u;   // before the first barrier
    constexpr int LPW = 5;                                  // K-tile loads per wave
    constexpr int EPI_STORES = E == Epi::Int32 ? 16 : 8;   // stores per wave after an epilogue
    constexpr int AHEAD = (NST - 2) * LPW;                  // loads younger than K-tile g + 1's
    issue(0);
#pragma unroll
    for (int i = 1; i < NST; ++i)
        if (i < total) issue(i);
    // K-tile 0 must have landed; every later prologue K-tile may still be in flight
    {
        const int later = (total < NST ? total : NST) - 1;
        if (later >= NST - 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm((NST - 1) * LPW));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    __syncthreads();
    read_frags(0, 0, 0);

    // End of K-tile g's first K-step: K-tile g+1 must have landed (at most the loads of K-tiles
    // g+2 .. g+NST-1 and, while the previous tile's epilogue stores are younger than K-tile
    // g+1's loads, those stores may still be in flight), then every wave has finished reading
    // stage g % NST, which takes K-tile g+NST; then K-tile g's second K-step.
    int g = 0;
    auto tail = [&](int t, int kt) {
        fence();
        if (g + NST - 1 < total) {
            if (t > 0 && kt < NST - 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(AHEAD + EPI_STORES));
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm(AHEAD));
        } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (g + NST < total) issue(g + NST);
        fence();
        // (after the stream's last K-tile this reads a stage whose fragments are never used)
        read_frags(g + 1, 0, 0);
        mfmas(1);
        interleave_reads();
        fence();
        ++g;
    };

    int gidx = 0;                                           // this stream's group index
    for (int t = 0; t < ntiles; ++t) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) facc[a][b] = v16f{};
        // group 0 of the tile: nothing to fold
        group_start(false, 0);
        read_frags(g, 1, 1);
        tail(t, 0);
        if constexpr (GKT == 2) {
            read_frags(g, 1, 1);
            mfmas(0);
            interleave_reads();
            tail(t, 1);
        }
        ++gidx;
        for (int gi = 1; gi < G; ++gi) {
            group_start(true, gidx - 1);
            read_frags(g, 1, 1);
            tail(t, GKT * gi);
            if constexpr (GKT == 2) {
                read_frags(g, 1, 1);
                mfmas(0);
                interleave_reads();
                tail(t, 2 * gi + 1);
            }
            ++gidx;
        }
        // the tile's last group, then its epilogue
        if (E == Epi::Bf16) read_scales(gidx - 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) fold_block(j >> 1, j & 1);
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

int64_t row_blocks(int64_t R) { return (R + 31) / 32; }

} // namespace

size_t w4a4_tiled_bytes(int64_t M, int64_t N, int K)
{
    return (size_t)(row_blocks(M) + row_blocks(N)) * (size_t)(K / 64) * PIECE;
}

hipError_t launch_tile_w4a4(const uint8_t *q, int64_t R, int K, uint8_t *out, hipStream_t stream)
{
    if (R <= 0) return hipSuccess;
    if (K % 128) return hipErrorInvalidValue;
    const int64_t units = row_blocks(R) * ((K + 255) / 256);  // 32 rows x 256 channels each
    if (units >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const int64_t want = (units + TILE_U - 1) / TILE_U;
    const int64_t grid = want < cu_count() * 8 ? want : cu_count() * 8;
    hipLaunchKernelGGL(tile_fp6_kernel, dim3((unsigned)grid), dim3(256), 0, stream, q, out, R, K, (uint32_t)units);
    return hipGetLastError();
}

hipError_t launch_gemm_w4a4(const uint8_t *xq, bool x_tiled, const uint8_t *wq, bool w_tiled, const uint16_t *sx,
                            const uint16_t *sw, const float *bias, void *y, Epi epi, int64_t M, int64_t N, int K,
                            int group, void *ws, hipStream_t stream)
{
    if (M <= 0 || N <= 0) return hipSuccess;
    // the epilogue's byte offset within a 32-row output block, 32 * N * 4 bytes at most, is 32-bit
    if (N >= ((int64_t)1 << 24)) return hipErrorInvalidValue;
    // the tile walk counts tiles in int
    if (((M + BM - 1) / BM) * ((N + BN - 1) / BN) >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    // scale groups of 2 K-tiles (256 channels) or 1 (128); at least 2 K-tiles (bias ring)
    const int gkt = group / BK;
    if ((gkt != 1 && gkt != 2) || K % group || K < 2 * BK) return hipErrorInvalidValue;
    uint8_t *xt_ws = static_cast<uint8_t *>(ws);
    const uint8_t *xt = xq;
    hipError_t e = hipSuccess;
    if (!x_tiled) {
        if ((e = launch_tile_w4a4(xq, M, K, xt_ws, stream)) != hipSuccess) return e;
        xt = xt_ws;
    }
    const uint8_t *wt = wq;
    if (!w_tiled) {
        uint8_t *wt_ws = xt_ws + row_blocks(M) * (K / 64) * PIECE;
        if ((e = launch_tile_w4a4(wq, N, K, wt_ws, stream)) != hipSuccess) return e;
        wt = wt_ws;
    }
    W4Params p;
    p.xt = xt;
    p.wt = wt;
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
    if (epi == Epi::Int32) {
        // the integer sums do not depend on the scale grouping
        if (gkt == 2) hipLaunchKernelGGL((gemm_w4a4_kernel<Epi::Int32, 2>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream, p);
        else hipLaunchKernelGGL((gemm_w4a4_kernel<Epi::Int32, 1>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream, p);
    } else if (gkt == 2) {
        hipLaunchKernelGGL((gemm_w4a4_kernel<Epi::Bf16, 2>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream, p);
    } else {
        hipLaunchKernelGGL((gemm_w4a4_kernel<Epi::Bf16, 1>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream, p);
    }
    return hipGetLastError();
}

} // namespace convrot
