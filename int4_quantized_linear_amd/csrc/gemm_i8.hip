// gemm_i8.hip -- INT8 x INT8 -> INT32 GEMM with the fused ConvRot dequant epilogue (gfx950).
//
//   acc[m,n] = sum_k xq[m,k] * wq[n,k]            (exact in int32 for K <= 133144)
//   y[m,n]   = bf16_rne(float(acc) * sx[m] * sw[n] + bias[n])
// xq: rotated, per-token INT8 activations [M,K]; wq: rotated, row-wise INT8 weights [N,K];
// both K-contiguous.  The rotation cancels in the product because R is orthogonal, so the
// integer GEMM runs on rotated codes directly and only the two scales are applied at the end
// ("minimax-h3-nvfp4-convrot核心原理", section 四: the INT8 tensor-core path is where ConvRot's
// speed comes from; "INT8 row-scale + ConvRot metadata").
//
// Design (MI355X / CDNA4):
//  * persistent: one 512-thread workgroup per CU walks a sequence of 256(M) x 256(N) output
//    tiles; the tiles of each XCD form a contiguous range of the tile order, walked in groups
//    along M so that the tiles running at the same time share their weight tile in that XCD's
//    L2.  8 wavefronts (2 per SIMD, so one covers the other's waits) in 2(N) x 4(M) each own a
//    128x64 sub-tile as 4x2 blocks of v_mfma_i32_32x32x32_i8 (128 int32 accumulators per lane,
//    about 230 of the 256 registers a wave has at 2 waves per SIMD, with no spills);
//  * K is streamed 128 bytes per K-tile through 2 LDS stages with buffer_load ... lds (global
//    -> LDS, no VGPRs).  A row's K-tile is one whole 128-byte cache line and one load
//    instruction moves 8 such lines, so every line is requested from L2 once (64-byte K-tiles
//    would request each line twice, in consecutive K-tiles).  The stream runs across tile
//    boundaries, so the next tile's first K-tiles load while the current tile finishes and
//    writes its epilogue.  Out-of-range rows and the K tail past K read through an
//    out-of-bounds buffer offset, which returns zeros;
//  * LDS rows are 128 bytes; 16-byte chunk c of row r sits at position c ^ ((r >> 1) & 7).
//    ds_read_b128 serves 16 lanes (256 bytes, all 64 banks) per cycle and a fragment read puts
//    16 consecutive rows on them: a row pair shares a 256-byte window and the XOR spreads the 8
//    pairs over distinct positions, so the reads are bank-conflict free;
//  * one barrier per K-tile, before its last MFMA sub-step: by then every wave has issued its
//    reads of this stage (fragments are read one sub-step ahead) and the next K-tile, issued a
//    whole K-tile earlier, has landed; the stage just read is then refilled with the K-tile
//    after next;
//  * the epilogue converts in registers and stores 16 bytes per lane straight to global memory
//    (lane pairs exchange halves with v_permlane32_swap so each store covers 8 columns); the
//    tile's sx/sw/bias are loaded into LDS with its first K-tile (4 rotating buffers: with short
//    K the load side can run up to 3 tiles ahead);
//  * split-K tail: when the tiles leave the grid's last round badly under-filled, the tail tiles
//    run as K-slices (the walk is over units: whole tiles, then slices), each slice storing its
//    exact int32 sums to a workspace slot, and split_reduce_kernel sums the slots and applies
//    the same epilogue arithmetic, so the outputs are bit-identical to the whole-tile path.
#include <type_traits>

#include "device_common.hpp"
#include "launchers.hpp"

namespace convrot {
namespace {

constexpr int BM = 256, BN = 256, BK = 128, NST = 2;
constexpr int OPB = 256 * BK;                 // bytes of one operand per stage (32 KiB)
constexpr int STAGE = 2 * OPB;                // weight rows then token rows
constexpr int SCALE_OFF = NST * STAGE;        // 128 KiB
constexpr int SCALE_BYTES = 4 * (2 * BN + BM);
constexpr int NSCALE = 4;
constexpr int SMEM = SCALE_OFF + NSCALE * SCALE_BYTES;
constexpr int NTHREADS = 512;
constexpr int GROUP_M = 4;
constexpr int WG_PER_CU = 1;
constexpr uint32_t OOB = 0x80000000u;         // buffer offset past num_records -> loads return 0
constexpr int NUM_RECORDS = 0x7ffffff0;

struct GemmParams {
    const int8_t *xq;
    const int8_t *wq;
    const float *sx;
    const float *sw;
    const float *bias;
    void *y;
    int64_t M, N;
    int K;
    int tiles_m, tiles_n;
    // Split-K tail: the first T_dp tiles of the tile order are computed whole; each of the r =
    // T - T_dp remaining tiles is computed as S K-slices, slice s of tail tile i writing its int32
    // partial sums to slot s*r + i of `part` (BM x BN int32, row-major); split_reduce_kernel sums
    // and dequantizes them.  S == 1: no split (T_dp == T).
    int32_t *part;
    int T_dp, S;
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= n only.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }

// Unit of virtual id pid (= blockIdx.x + k * gridDim.x, gridDim.x a multiple of 8).  Dispatch ids
// are spread round-robin over the 8 XCDs, so pid keeps its XCD.  Units 0..T_dp-1 are the whole
// tiles, then come the split units; each XCD walks a contiguous range of the whole tiles, then a
// contiguous range of the split units (T_dp is a multiple of 8 whenever there are split units, so
// this is a bijection of [0, U)).
__device__ __forceinline__ int unit_of(int pid, int T_dp, int U)
{
    const int xcd = pid & 7, local = pid >> 3;
    const int dper = T_dp >> 3, drem = T_dp & 7;
    const int dn = dper + (xcd < drem);
    if (local < dn) return xcd * dper + min(xcd, drem) + local;
    const int ut = U - T_dp, tper = ut >> 3, trem = ut & 7;
    return T_dp + xcd * tper + min(xcd, trem) + (local - dn);
}

// Tile q of the M-grouped order: groups of GROUP_M tile rows, walked column by column, so the
// tiles an XCD runs at the same time share their weight tiles in its L2.
__device__ __forceinline__ void tile_coords(int q, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int span = GROUP_M * tiles_n;
    const int first_m = (q / span) * GROUP_M;
    const int gsz = min(tiles_m - first_m, GROUP_M);
    const int r = q % span;
    tm = first_m + r % gsz;
    tn = r / gsz;
}

template <Epi E, bool VEC>
__global__ void __launch_bounds__(NTHREADS, WG_PER_CU) gemm_i8_kernel(GemmParams p)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wn = w & 1, wm = w >> 1;   // wn: 128-row half of N, wm: 64-row quarter of M
    const int K = p.K;
    const int KT = (K + BK - 1) / BK;          // the last K-tile may be half (K % 128 == 64)
    const int T = p.tiles_m * p.tiles_n;
    const int U = p.T_dp + (T - p.T_dp) * p.S;
    // jobs of this workgroup: virtual ids blockIdx.x + j*gridDim.x < U.  Job j is a unit: tile
    // (tm, tn), its K-tiles [kb, ke), and the partial-sum slot of a split unit (-1: whole tile).
    const int njobs = (U - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    struct Job {
        int tm, tn, kb, ke, slot;
    };
    auto job = [&](int j) {
        Job J;
        const int u = unit_of((int)blockIdx.x + j * (int)gridDim.x, p.T_dp, U);
        int q = u;
        J.kb = 0;
        J.ke = KT;
        J.slot = -1;
        if (u >= p.T_dp) {
            // slice-major: the units an XCD runs at once are neighbouring tiles at the same K-slice,
            // so they share operand rows in its L2 like whole tiles do
            const int r = T - p.T_dp, v = u - p.T_dp, sl = v / r;
            q = p.T_dp + v % r;
            J.kb = sl * KT / p.S;
            J.ke = (sl + 1) * KT / p.S;
            J.slot = v;
        }
        tile_coords(q, p.tiles_m, p.tiles_n, J.tm, J.tn);
        return J;
    };
    int total = 0;                            // K-tiles in this workgroup's stream
    for (int j = 0; j < njobs; ++j) {
        const Job J = job(j);
        total += J.ke - J.kb;
    }

    // Per-lane load geometry (independent of the tile): instruction i (0..3) of wave w fills
    // LDS rows 8*(8i+w) .. +7 of an operand stage; lane -> row +lane/8 at 16-byte position
    // lane%8, which holds K chunk (lane%8) ^ swz(row).
    int lrow[4], lchunk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        lrow[i] = 8 * (8 * i + w) + (lane >> 3);
        lchunk[i] = (lane & 7) ^ swz(lrow[i]);
    }

    // Current load-side tile (the stream runs ahead of the compute-side tile).
    int ld_tm = 0, ld_tn = 0;
    __amdgpu_buffer_rsrc_t rw, rx;
    uint32_t offw[4], offx[4];
    auto set_load_tile = [&](int tm, int tn) {
        ld_tm = tm;
        ld_tn = tn;
        const int64_t m0 = (int64_t)ld_tm * BM, n0 = (int64_t)ld_tn * BN;
        rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(p.wq + n0 * K), (short)0, NUM_RECORDS, 0x00020000);
        rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(p.xq + m0 * K), (short)0, NUM_RECORDS, 0x00020000);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t o = (uint32_t)(lrow[i] * K + 16 * lchunk[i]);
            offw[i] = n0 + lrow[i] < p.N ? o : OOB;
            offx[i] = m0 + lrow[i] < p.M ? o : OOB;
        }
    };
    // The tile's sw, bias and sx (256 floats each) go to LDS scale buffer (t & 3) with the
    // tile's first K-tile: 12 dword load-to-LDS instructions, 2 on each of waves 0-5.
    // Out-of-range entries and a missing bias read as zeros.
    auto issue_scales = [&](int t) {
        if constexpr (E == Epi::Bf16) {
            const int64_t m0 = (int64_t)ld_tm * BM, n0 = (int64_t)ld_tn * BN;
            const int64_t nrem = p.N - n0, mrem = p.M - m0;
            const __amdgpu_buffer_rsrc_t rs[3] = {
                __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p.sw + n0), (short)0, (int)(4 * (nrem < BN ? nrem : BN)), 0x00020000),
                __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p.bias ? p.bias + n0 : p.sw), (short)0,
                                                  p.bias ? (int)(4 * (nrem < BN ? nrem : BN)) : 0, 0x00020000),
                __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p.sx + m0), (short)0, (int)(4 * (mrem < BM ? mrem : BM)), 0x00020000)};
            uint8_t *sb = smem + SCALE_OFF + (t & (NSCALE - 1)) * SCALE_BYTES;
            if (w < 6) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int a = 2 * w + j, arr = a >> 2, part = a & 3;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[arr], (lds_void *)(sb + arr * 1024 + part * 256), 4,
                                                             (uint32_t)(part * 256 + 4 * lane), 0, 0, 0);
                }
            }
        }
    };
    // Issue the loads of the next K-tile of the stream (8 buffer_load ... lds per wave, plus the
    // scales with a tile's first K-tile) into LDS stage (g & 1).  The load side walks the stream
    // in order: K-tile ld_kt of job ld_j is the one it issues next.
    // The K position goes in the scalar offset, so a K-tile costs no VALU: an out-of-range row's
    // lane offset (OOB) stays past num_records with any K added.  Only a half K-tile at the end
    // of K (K % 128 == 64) needs per-lane offsets, to read zeros for the chunks past K.
    int ld_j = -1, ld_kt = 0, ld_ke = 0;
    const bool khalf = (K % BK) != 0;
    auto issue = [&](int g) {
        if (ld_kt == ld_ke) {
            const Job J = job(++ld_j);
            set_load_tile(J.tm, J.tn);
            issue_scales(ld_j);
            ld_kt = J.kb;
            ld_ke = J.ke;
        }
        const int k0 = __builtin_amdgcn_readfirstlane(ld_kt * BK);
        const bool tail = khalf && ld_kt == KT - 1;
        ++ld_kt;
        uint8_t *base = smem + (g & (NST - 1)) * STAGE + w * 1024;
        if (!tail) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(base + 8 * i * 1024), 16, offw[i], k0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(base + OPB + 8 * i * 1024), 16, offx[i], k0, 0, 0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool kin = lchunk[i] < (BK / 2) / 16;              // chunks 0..3 exist
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(base + 8 * i * 1024), 16,
                                                         kin ? offw[i] : OOB, k0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(base + OPB + 8 * i * 1024), 16,
                                                         kin ? offx[i] : OOB, k0, 0, 0);
            }
        }
    };

    // Fragment addressing: row = wave base + 32*blk + lane%32 (bases are multiples of 32, so
    // swz(row) == swz(lane%32)); sub-step kk (0..3) reads K chunk 2*kk + lane/32.
    const int frow = lane & 31, fhalf = lane >> 5;
    const int arow = (wn * 128 + frow) * BK, brow = OPB + (wm * 64 + frow) * BK;
    const int fpos[4] = {((0 + fhalf) ^ swz(frow)) * 16, ((2 + fhalf) ^ swz(frow)) * 16,
                         ((4 + fhalf) ^ swz(frow)) * 16, ((6 + fhalf) ^ swz(frow)) * 16};
    v4i fa[2][4], fb[2][2];
    auto read_frags = [&](int g, int kk, int buf) {
        const uint8_t *s0 = smem + (g & (NST - 1)) * STAGE + fpos[kk];
#pragma unroll
        for (int b = 0; b < 4; ++b) fa[buf][b] = *reinterpret_cast<const v4i *>(s0 + arow + 32 * b * BK);
#pragma unroll
        for (int b = 0; b < 2; ++b) fb[buf][b] = *reinterpret_cast<const v4i *>(s0 + brow + 32 * b * BK);
    };
    v16i acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = v16i{};
    auto mfma_range = [&](int buf, int j0, int j1) {
#pragma unroll
        for (int j = j0; j < j1; ++j) {
            const int bi = j >> 1, bj = j & 1;
            acc[bi][bj] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[buf][bi], fb[buf][bj], acc[bi][bj], 0, 0, 0);
        }
    };
    auto mfmas = [&](int buf) { mfma_range(buf, 0, 8); };
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

    // Accumulator layout of a 32x32 block (MFMA rows = weight rows n, columns = tokens m):
    // lane holds m = lane%32 and, for register v, n = 8*(v/4) + 4*(lane/32) + v%4.
    // Stores go through a buffer descriptor per 32-row block (uniform, in SGPRs) with 32-bit
    // lane offsets; out-of-range rows/columns get an out-of-bounds offset and are dropped.  This
    // keeps the epilogue's register footprint small: a spill reload here would wait on vmcnt
    // and so drain every store and prefetch in flight.
    auto epilogue = [&](const Job &J, int j) {
        const int m0 = J.tm * BM, n0 = J.tn * BN;
        const int Mi = (int)p.M, Ni = (int)p.N;
        // lane-dependent bases laundered so the addresses below are formed here, not hoisted out
        // of the tile loop (where they would stay live through the main loop)
        int erow = frow, ecol = wn * 128 + 4 * fhalf;
        asm volatile("" : "+v"(erow), "+v"(ecol));
        if constexpr (E == Epi::Int32) {
#pragma unroll
            for (int bj = 0; bj < 2; ++bj) {
                const int mr = m0 + wm * 64 + 32 * bj;            // first row of the block (uniform)
                const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
                    static_cast<int32_t *>(p.y) + (int64_t)mr * p.N, (short)0, NUM_RECORDS, 0x00020000);
                const bool rok = mr + erow < Mi;
#pragma unroll
                for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int n = n0 + ecol + 32 * bi + 8 * g;
                        const v4u d = {(unsigned)acc[bi][bj][4 * g], (unsigned)acc[bi][bj][4 * g + 1],
                                       (unsigned)acc[bi][bj][4 * g + 2], (unsigned)acc[bi][bj][4 * g + 3]};
                        if (VEC || n + 3 < Ni) {
                            const uint32_t off = (rok && n < Ni) ? (uint32_t)(erow * Ni + n) * 4u : OOB;
                            __builtin_amdgcn_raw_buffer_store_b128(d, ry, off, 0, 0);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const uint32_t off = (rok && n + e < Ni) ? (uint32_t)(erow * Ni + n + e) * 4u : OOB;
                                __builtin_amdgcn_raw_buffer_store_b32(d[e], ry, off, 0, 0);
                            }
                        }
                    }
                fence();
            }
        } else if (VEC && J.slot >= 0) {
            // split unit (16-byte-store variant only): its int32 partial sums go to slot J.slot
            // (BM x BN int32, row-major).  Rows past M and column groups past N are not written,
            // and never read.
            int32_t *slot = p.part + (int64_t)J.slot * (BM * BN);
            // own laundered lane bases, so that no address of this branch is shared with (and kept
            // live across) the bf16 branch
            int prow = frow, pcol = wn * 128 + 4 * fhalf;
            asm volatile("" : "+v"(prow), "+v"(pcol));
#pragma unroll
            for (int bj = 0; bj < 2; ++bj) {
                const int ml = wm * 64 + 32 * bj;
                const __amdgpu_buffer_rsrc_t rp =
                    __builtin_amdgcn_make_buffer_rsrc(slot + ml * BN, (short)0, NUM_RECORDS, 0x00020000);
                const bool rok = m0 + ml + prow < Mi;
#pragma unroll
                for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int nl = pcol + 32 * bi + 8 * g;
                        const v4u d = {(unsigned)acc[bi][bj][4 * g], (unsigned)acc[bi][bj][4 * g + 1],
                                       (unsigned)acc[bi][bj][4 * g + 2], (unsigned)acc[bi][bj][4 * g + 3]};
                        const uint32_t off = (rok && n0 + nl < Ni) ? (uint32_t)(prow * BN + nl) * 4u : OOB;
                        __builtin_amdgcn_raw_buffer_store_b128(d, rp, off, 0, 0);
                    }
                fence();
            }
        } else {
            const float *ls = reinterpret_cast<const float *>(smem + SCALE_OFF + (j & (NSCALE - 1)) * SCALE_BYTES);
#pragma unroll
            for (int bj = 0; bj < 2; ++bj) {
                const int mr = m0 + wm * 64 + 32 * bj;
                const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
                    static_cast<uint16_t *>(p.y) + (int64_t)mr * p.N, (short)0, NUM_RECORDS, 0x00020000);
                const bool rok = mr + erow < Mi;
                const float sxm = ls[2 * BN + wm * 64 + 32 * bj + erow];
#pragma unroll
                for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                    for (int g2 = 0; g2 < 2; ++g2) {
                        // column groups g = 2*g2 and 2*g2+1 of block bi: 4 columns each per lane
                        uint32_t pk[2][2];
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int g = 2 * g2 + h;
                            const int nl = ecol + 32 * bi + 8 * g;
                            const v4f s4 = *reinterpret_cast<const v4f *>(ls + nl);
                            const v4f b4 = *reinterpret_cast<const v4f *>(ls + BN + nl);
                            float yv[4];
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                yv[i] = __builtin_fmaf((float)acc[bi][bj][4 * g + i], sxm * s4[i], b4[i]);
                            pk[h][0] = pack_bf16x2(yv[0], yv[1]);
                            pk[h][1] = pack_bf16x2(yv[2], yv[3]);
                        }
                        // lane l < 32 now gets columns 8g..8g+7 of group g = 2*g2, lane l+32 those
                        // of group 2*g2+1 (same token row m)
                        swap32(pk[0][0], pk[1][0]);
                        swap32(pk[0][1], pk[1][1]);
                        const int n = n0 + (ecol - 4 * fhalf) + 32 * bi + 8 * (2 * g2 + fhalf);
                        if constexpr (VEC) {
                            const uint32_t off = (rok && n < Ni) ? (uint32_t)(erow * Ni + n) * 2u : OOB;
                            __builtin_amdgcn_raw_buffer_store_b128(v4u{pk[0][0], pk[0][1], pk[1][0], pk[1][1]}, ry, off, 0, 0);
                        } else {
                            // rows not 16-byte aligned (N % 8 != 0): element stores, clipped at N
                            const uint32_t wv[4] = {pk[0][0], pk[0][1], pk[1][0], pk[1][1]};
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const uint32_t off = (rok && n + e < Ni) ? (uint32_t)(erow * Ni + n + e) * 2u : OOB;
                                __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(wv[e >> 1] >> (16 * (e & 1))), ry, off, 0, 0);
                            }
                        }
                    }
                fence();
            }
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) acc[a][b] = v16i{};
    };

    if (njobs <= 0) return;
    // Stores each wavefront has in flight after an epilogue (vmcnt counts them too; a split
    // unit's partial epilogue issues 32, so the wait after it is a little stricter than needed).
    constexpr int EPI_STORES = E == Epi::Int32 ? 32 : 16;
    // prologue: K-tile 0 (and tile 0's scales) visible, K-tile 1 in flight, first fragments
    issue(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    if (total > 1) issue(1);
    read_frags(0, 0, 0);

    int g = 0;
    for (int j = 0; j < njobs; ++j) {
        const Job J = job(j);
        for (int kt = J.kb; kt < J.ke; ++kt, ++g) {
            read_frags(g, 1, 1);
            fence();
            mfmas(0);
            fence();
            read_frags(g, 2, 0);
            fence();
            mfmas(1);
            fence();
            read_frags(g, 3, 1);
            fence();
            mfmas(0);
            fence();
            // K-tile g+1 must have landed before its first fragments are read.  Issued after
            // its loads: at most the previous tile's epilogue stores, right after an epilogue
            // (and only with 16-byte stores; otherwise wait for everything).
            if (g + 1 < total) {
                if (VEC && j > 0 && kt == J.kb) __builtin_amdgcn_s_waitcnt(waitcnt_vm(EPI_STORES));
                else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            }
            // Every wave has completed (lgkmcnt(0)) its reads of stage g & 1 and waited for its
            // loads of K-tile g+1.  A raw barrier: the fence of __syncthreads() would make the
            // compiler wait for every store in flight as well.
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            // last sub-step: the loads of K-tile g+2 and the first fragments of g+1 are issued
            // between its MFMAs, so the matrix pipe is fed while they go out
            mfma_range(1, 0, 2);
            fence();
            if (g + 2 < total) issue(g + 2);
            fence();
            mfma_range(1, 2, 4);
            fence();
            if (g + 1 < total) read_frags(g + 1, 0, 0);
            fence();
            mfma_range(1, 4, 8);
            fence();
        }
        epilogue(J, j);
    }
}

// Split-K tail, second pass: for each split tile, sum its S int32 partial slots (exact, in any
// order) and apply the same epilogue arithmetic as gemm_i8_kernel, fma(float(acc), sx*sw, bias)
// then bf16 RNE, so a split tile's outputs are bit-identical to a whole tile's.  A thread owns 8
// consecutive columns of one row (N % 8 == 0, so all 8 exist; 32 threads cover a row's 256 columns) and a 256-thread
// workgroup 8 rows; rb workgroups cover the rows of a tile that exist (all 256 unless M < 256).
// All S slices' loads are issued before the first add.
constexpr int MAX_SPLIT = 8;
struct ReduceParams {
    const int32_t *part;
    const float *sx;
    const float *sw;
    const float *bias;
    uint16_t *y;
    int64_t M, N;
    int tiles_m, tiles_n;
    int T_dp, S, rb;
};

__global__ void __launch_bounds__(256) split_reduce_kernel(ReduceParams p)
{
    const int i = (int)blockIdx.x / p.rb;                               // tail tile
    const int ml = ((int)blockIdx.x % p.rb) * 8 + ((int)threadIdx.x >> 5);
    const int nl = ((int)threadIdx.x & 31) * 8;
    int tm, tn;
    tile_coords(p.T_dp + i, p.tiles_m, p.tiles_n, tm, tn);
    const int64_t m = (int64_t)tm * BM + ml, n = (int64_t)tn * BN + nl;
    if (m >= p.M || n >= p.N) return;
    const int r = p.tiles_m * p.tiles_n - p.T_dp;
    v4i a[MAX_SPLIT], b[MAX_SPLIT];
#pragma unroll
    for (int s = 0; s < MAX_SPLIT; ++s) {
        if (s < p.S) {
            const int32_t *src = p.part + ((int64_t)s * r + i) * (BM * BN) + ml * BN + nl;
            a[s] = *reinterpret_cast<const v4i *>(src);
            b[s] = *reinterpret_cast<const v4i *>(src + 4);
        }
    }
    int32_t sum[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < MAX_SPLIT; ++s) {
        if (s < p.S) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sum[e] += a[s][e];
                sum[e + 4] += b[s][e];
            }
        }
    }
    const float sxm = p.sx[m];
    float yv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        yv[e] = __builtin_fmaf((float)sum[e], sxm * p.sw[n + e], p.bias ? p.bias[n + e] : 0.0f);
    uint32_t pk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(yv[2 * e], yv[2 * e + 1]);
    *reinterpret_cast<v4u *>(p.y + m * p.N + n) = v4u{pk[0], pk[1], pk[2], pk[3]};
}

int cu_count_cached()
{
    static int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            n = 256;
        return n > 0 ? n : 256;
    }();
    return cus;
}

// Persistent grid capacity: workgroups that run at once, a multiple of 8 (XCD count) so that
// virtual ids keep their XCD.
int grid_capacity() { return ((cu_count_cached() * WG_PER_CU) & ~7) > 0 ? (cu_count_cached() * WG_PER_CU) & ~7 : 8; }

struct SplitPlan {
    int T_dp, S;
    size_t bytes;
};

// When the tiles leave the last round of the persistent grid partly idle (T % capacity = r > 0),
// the r tail tiles may be split into S K-slices (S <= 8, each at least 2 K-tiles) so that the
// tail spreads over more CUs.  The kernel is power-bound when most CUs run: a K-tile of a tile
// takes ~1.84 us with every CU busy, but ~1.38 us when fewer than ~3/4 of them are (higher
// clocks; measured on the prefill and the 160-tile shapes).  So a round of n units of L K-tiles
// takes L * max(1.38 us, n * 1.84 us / capacity), and spreading a tail that already keeps ~3/4
// of the CUs busy gains little.  Against that: the partial sums' round trip (8 bytes per output
// element of the tail and slice, counted at 2.5 TB/s: each unit's int32 stores leave in a burst at
// its end, and a q|k|v-shaped tail of 64 tiles in 3 slices measured no faster than whole) and the
// second launch.  A split is planned only if it saves at least 5% of the estimated GEMM time.
SplitPlan plan_split(int64_t M, int64_t N, int K)
{
    const int64_t tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const int64_t T = tiles_m * tiles_n;
    const int cap = grid_capacity();
    SplitPlan pl = {(int)T, 1, 0};
    const int64_t full = T / cap, r = T % cap;
    // only the 16-byte-store variant (N % 8 == 0) has the partial-sum epilogue
    if (r == 0 || N % 8 != 0 || T >= ((int64_t)1 << 30)) return pl;
    const int KT = (K + BK - 1) / BK;
    const double t_full = 1.84e-6, t_fast = 1.38e-6;
    const double rows = (double)(M < BM ? M : BM);
    auto tail_time = [&](int S) {
        const double power = (double)r * KT * t_full / cap;
        const double rounds = (double)((r * S + cap - 1) / cap);
        const double clock = rounds * ((double)KT / S) * t_fast;
        return power > clock ? power : clock;
    };
    const double whole = (double)full * KT * t_full + tail_time(1);
    double best = tail_time(1);
    for (int S = 2; S <= MAX_SPLIT && KT / S >= 2; ++S) {
        const double t = tail_time(S) + (double)(r * S) * rows * BN * 8.0 / 2.5e12 + 4e-6;
        if (t < best && tail_time(1) - t >= 0.05 * whole) {
            best = t;
            pl = {(int)(full * cap), S, (size_t)(r * S) * BM * BN * sizeof(int32_t)};
        }
    }
    return pl;
}

} // namespace

size_t gemm_i8_split_bytes(int64_t M, int64_t N, int K)
{
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    return plan_split(M, N, K).bytes;
}

hipError_t launch_gemm_i8(const int8_t *xq, const int8_t *wq, const float *sx, const float *sw, const float *bias,
                          void *y, Epi epi, int64_t M, int64_t N, int K, void *part, size_t part_bytes,
                          hipStream_t stream)
{
    if (M <= 0 || N <= 0) return hipSuccess;
    // the epilogue's byte offset within a 32-row output block, 32 * N * 4 bytes at most, is 32-bit
    if (N >= ((int64_t)1 << 24)) return hipErrorInvalidValue;
    GemmParams p;
    p.xq = xq;
    p.wq = wq;
    p.sx = sx;
    p.sw = sw;
    p.bias = bias;
    p.y = y;
    p.M = M;
    p.N = N;
    p.K = K;
    // the tile walk counts tiles in int
    if (((M + BM - 1) / BM) * ((N + BN - 1) / BN) >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    p.tiles_m = (int)((M + BM - 1) / BM);
    p.tiles_n = (int)((N + BN - 1) / BN);
    const int T = p.tiles_m * p.tiles_n;
    // split-K tail (bf16 output only, and only with room for the partial sums)
    SplitPlan pl = {T, 1, 0};
    if (epi == Epi::Bf16 && part) {
        pl = plan_split(M, N, K);
        if (pl.S > 1 && part_bytes < pl.bytes) pl = {T, 1, 0};
    }
    p.part = static_cast<int32_t *>(part);
    p.T_dp = pl.T_dp;
    p.S = pl.S;
    const int U = pl.T_dp + (T - pl.T_dp) * pl.S;
    // persistent grid: a multiple of 8 (XCD count) so virtual ids keep their XCD
    int grid = grid_capacity();
    if (U < grid) grid = (U + 7) & ~7;
    if (epi == Epi::Int32)
        hipLaunchKernelGGL((gemm_i8_kernel<Epi::Int32, true>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream, p);
    else if (N % 8 == 0)
        hipLaunchKernelGGL((gemm_i8_kernel<Epi::Bf16, true>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream, p);
    else
        hipLaunchKernelGGL((gemm_i8_kernel<Epi::Bf16, false>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || pl.S == 1) return e;
    ReduceParams r;
    r.part = p.part;
    r.sx = sx;
    r.sw = sw;
    r.bias = bias;
    r.y = static_cast<uint16_t *>(y);
    r.M = M;
    r.N = N;
    r.tiles_m = p.tiles_m;
    r.tiles_n = p.tiles_n;
    r.T_dp = pl.T_dp;
    r.S = pl.S;
    r.rb = (int)((M < BM ? M : BM) + 7) / 8;
    const unsigned rgrid = (unsigned)(T - pl.T_dp) * (unsigned)r.rb;
    hipLaunchKernelGGL(split_reduce_kernel, dim3(rgrid), dim3(256), 0, stream, r);
    return hipGetLastError();
}

} // namespace convrot
