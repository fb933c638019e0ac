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
//    128x64 sub-tile as 8x4 blocks of v_mfma_i32_16x16x64_i8 (128 int32 accumulators per lane,
//    255 of the 256 registers a wave has at 2 waves per SIMD, with no spills).  On gfx950 the
//    16x16x64 form sustains more operations per second than the 32x32x32 one (4.4-4.5 against
//    3.8 POP/s in register-only loops) for the same fragment bytes per operation;
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
//  * the epilogue converts in registers, passes each 32-row block through LDS and stores whole
//    rows of 256 bytes (N % 8 == 0; element stores otherwise); the tile's sx/sw/bias are loaded
//    into LDS with its first K-tile (4 rotating buffers: with short K the load side can run up
//    to 3 tiles ahead);
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
// 1 KiB per wave that a K-tile's loads target when they are not issued for real (the last
// K-tile of a job, whose stage the epilogue uses first): out-of-range zeros land here
constexpr int DUMMY_OFF = SCALE_OFF + NSCALE * SCALE_BYTES;
constexpr int SMEM = DUMMY_OFF + 8 * 1024;
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
    int M, N;                  // < 2^31 (checked by the C-ABI layer)
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

// Buffer descriptor from a wave-uniform address and size, built from readfirstlane'd halves so it
// stays in scalar registers.  (readfirstlane returns int: each half goes through uint32_t, so the
// low half is zero-extended, not sign-extended, into the 64-bit address.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(uint64_t a, int bytes)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | (uint64_t)lo), (short)0,
                                             __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

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
    // The tile's operand bases are kept as integers and made into buffer descriptors at each
    // use from readfirstlane'd halves: they are uniform, and a descriptor value carried through
    // the loop's job switch could otherwise be placed in VGPRs, which turns every load into a
    // waterfall loop.
    int ld_tm = 0, ld_tn = 0;
    uint64_t wbase_addr = 0, xbase_addr = 0;
    uint32_t offw[4], offx[4];
    auto set_load_tile = [&](int tm, int tn) {
        ld_tm = tm;
        ld_tn = tn;
        const int64_t m0 = (int64_t)ld_tm * BM, n0 = (int64_t)ld_tn * BN;
        wbase_addr = reinterpret_cast<uint64_t>(p.wq + n0 * K);
        xbase_addr = reinterpret_cast<uint64_t>(p.xq + m0 * K);
        // rows left in the operands past the tile's first row (32-bit: N, M < 2^31)
        const int nrem = __builtin_amdgcn_readfirstlane(p.N - ld_tn * BN);
        const int mrem = __builtin_amdgcn_readfirstlane(p.M - ld_tm * BM);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t o = (uint32_t)(lrow[i] * K + 16 * lchunk[i]);
            offw[i] = lrow[i] < nrem ? o : OOB;
            offx[i] = lrow[i] < mrem ? o : OOB;
        }
    };
    // The tile's sw, bias and sx (256 floats each) go to LDS scale buffer (t & 3) with the
    // tile's first K-tile: 12 dword load-to-LDS instructions, 2 on each of waves 0-5.
    // Out-of-range entries and a missing bias read as zeros.
    auto issue_scales = [&](int t) {
        if constexpr (E == Epi::Bf16) {
            const int64_t m0 = (int64_t)ld_tm * BM, n0 = (int64_t)ld_tn * BN;
            const int nb = (int)(4 * (p.N - n0 < BN ? p.N - n0 : BN)), mb = (int)(4 * (p.M - m0 < BM ? p.M - m0 : BM));
            uint8_t *sb = smem + SCALE_OFF + (t & (NSCALE - 1)) * SCALE_BYTES;
            if (w < 6) {
                // array arr = w / 2 (0 sw, 1 bias, 2 sx), picked with wave-uniform scalars so the
                // descriptor stays in SGPRs
                const int arr = w >> 1;
                const float *src = arr == 0 ? p.sw + n0 : arr == 1 ? (p.bias ? p.bias + n0 : p.sw) : p.sx + m0;
                const int bytes = arr == 0 ? nb : arr == 1 ? (p.bias ? nb : 0) : mb;
                const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(reinterpret_cast<uint64_t>(src), bytes);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int part = (2 * w + j) & 3;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(sb + arr * 1024 + part * 256), 4,
                                                             (uint32_t)(part * 256 + 4 * lane), 0, 0, 0);
                }
            }
        }
    };
    // Load side of the stream.  K-tile ld_kt of job ld_j is the next one it issues, from the
    // descriptors set by set_load_tile.  issue_ktile() is straight-line code (8 buffer_load ... lds
    // per wave into LDS stage g & 1, no branch), so the scheduler can spread the loads between
    // MFMAs; the K position goes in the scalar offset, so a K-tile costs no VALU beyond two selects
    // per load: chunks past K of a half K-tile at the end of K (K % 128 == 64) and every load once
    // the stream is exhausted get an out-of-range offset (zeros land in LDS, no memory access).
    // next_job() moves the load side to the next job when a job's K-tiles have all been issued;
    // it runs once per job, outside the MFMA-interleaved region, and issues the job's scales then.
    int ld_j = -1, ld_kt = 0, ld_ke = 0;
    uint32_t ld_done = 0u;                    // OOB once every K-tile of the stream has been issued
    const bool khalf = (K % BK) != 0;
    uint32_t tmask[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) tmask[i] = lchunk[i] >= (BK / 2) / 16 ? OOB : 0u;   // chunks 4..7: past K
    // (The load-side counters are uniform; readfirstlane states it, so that they and the branch
    // on them stay scalar.)
    auto next_job = [&]() __attribute__((always_inline)) {
        ld_j = __builtin_amdgcn_readfirstlane(ld_j + 1);
        // (assigned outside the branch: two branches that each store one counter get merged into
        // one store through a pointer select, which keeps the counters in scratch memory)
        ld_done = ld_j < njobs ? 0u : OOB;
        if (ld_j < njobs) {
            const Job J = job(ld_j);
            set_load_tile(J.tm, J.tn);
            issue_scales(ld_j);
            ld_kt = __builtin_amdgcn_readfirstlane(J.kb);
            ld_ke = __builtin_amdgcn_readfirstlane(J.ke);
        }
    };
    // real == false (the last K-tile of a job): the same instructions, but out of range into the
    // wave's dummy 1 KiB, and the stream does not advance; the epilogue issues the K-tile for real
    // once it is done with the stage.  (A uniform select rather than a branch keeps one copy of
    // the MFMA-interleaved region.)
    auto issue_ktile = [&](int g, bool real) __attribute__((always_inline)) {
        const int k0 = __builtin_amdgcn_readfirstlane(ld_kt * BK);
        const uint32_t tsel = (khalf && ld_kt == KT - 1) ? 0xffffffffu : 0u;
        uint8_t *base = smem + (g & (NST - 1)) * STAGE + w * 1024;
        uint8_t *dummy = smem + DUMMY_OFF + w * 1024;
        const uint32_t skip = real ? 0u : OOB;
        const __amdgpu_buffer_rsrc_t rw = uniform_rsrc(wbase_addr, NUM_RECORDS), rx = uniform_rsrc(xbase_addr, NUM_RECORDS);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t extra = (tmask[i] & tsel) | ld_done | skip;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(real ? base + 8 * i * 1024 : dummy), 16,
                                                     offw[i] | extra, k0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(real ? base + OPB + 8 * i * 1024 : dummy), 16,
                                                     offx[i] | extra, k0, 0, 0);
        }
        ld_kt = __builtin_amdgcn_readfirstlane(ld_kt + (real ? 1 : 0));
    };

    // Fragment addressing (16x16x64 blocks): lane l supplies row (block base) + l%16 and the 16
    // bytes of K chunk 4*kk + l/16 in K-step kk (0..1) of the K-tile; A and B use the same chunk
    // for a lane, so every channel of the K-step meets its partner once.  Block bases are multiples
    // of 16, so swz(row) == swz(l%16).
    const int frow = lane & 15, fq = lane >> 4;
    const int arow = (wn * 128 + frow) * BK, brow = OPB + (wm * 64 + frow) * BK;
    const int fpos[2] = {((0 + fq) ^ swz(frow)) * 16, ((4 + fq) ^ swz(frow)) * 16};
    // fa[h]: weight blocks 4h..4h+3 of the K-step being worked on; fb[kk]: the 4 token blocks of
    // K-step kk.  A K-tile runs as 4 sub-steps (kk, h) of 16 MFMAs each, in the order (0,0), (0,1),
    // (1,0), (1,1); each sub-step reads the fragments the next one needs into the registers its
    // predecessor has finished with.
    v4i fa[2][4], fb[2][4];
    auto read_a = [&](int g, int kk, int h) {
        const uint8_t *s0 = smem + (g & (NST - 1)) * STAGE + fpos[kk] + arow;
#pragma unroll
        for (int b = 0; b < 4; ++b) fa[h][b] = *reinterpret_cast<const v4i *>(s0 + 16 * (4 * h + b) * BK);
    };
    auto read_b = [&](int g, int kk) {
        const uint8_t *s0 = smem + (g & (NST - 1)) * STAGE + fpos[kk] + brow;
#pragma unroll
        for (int b = 0; b < 4; ++b) fb[kk][b] = *reinterpret_cast<const v4i *>(s0 + 16 * b * BK);
    };
    v4i acc[8][4];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = v4i{};
    auto mfma_range = [&](int kk, int h, int j0, int j1) {
#pragma unroll
        for (int j = j0; j < j1; ++j) {
            const int bi = 4 * h + (j >> 2), bj = j & 3;
            acc[bi][bj] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[h][j >> 2], fb[kk][bj], acc[bi][bj], 0, 0, 0);
        }
    };
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

    // Accumulator layout of a 16x16 block (MFMA rows = weight rows n, columns = tokens m):
    // lane holds m = lane%16 and, for register v, n = 4*(lane/16) + v.
    // Stores go through a buffer descriptor per block of output rows (16, or 32 for the bf16
    // 16-byte-store variant; uniform, in SGPRs) with 32-bit lane offsets; out-of-range
    // rows/columns get an out-of-bounds offset and are dropped.  This keeps the epilogue's
    // register footprint small: a spill reload here would wait on vmcnt and so drain every store
    // and prefetch in flight.
    // The epilogue of a job runs after its last K-tile g.  It issues the loads of K-tile g + 2 (in
    // the K loop they go out during the last sub-step; for a job's last K-tile they wait until
    // here) before its stores (the bf16 16-byte-store variant: before its last row block's), so
    // that the first barrier of the next job can leave those stores in flight.  That variant
    // passes each 32-row block through the wave's own 8 KiB of the LDS stage K-tile g occupied
    // (every wave has read it: barrier of K-tile g) -- exactly the 8 pieces of 1 KiB this wave's
    // loads of K-tile g + 2 refill, so no other wave touches them -- and writes whole 128-byte
    // lines: 4 rows x 256 bytes per store instruction rather than the 8-byte pieces of one row
    // that each lane holds.
    auto issue_after_epilogue_reads = [&](int g) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // LDS reads of the region done
        issue_ktile(g, true);
        if (ld_kt == ld_ke) next_job();
    };
    auto epilogue = [&](const Job &J, int j, int g) {
        const int m0 = J.tm * BM, n0 = J.tn * BN;
        const int Mi = p.M, Ni = p.N;
        // lane-dependent bases laundered so the addresses below are formed here, not hoisted out
        // of the tile loop (where they would stay live through the main loop): the lane's token
        // row in a 16-row block and its first weight column in a 16-column block
        int erow = frow, ecol = wn * 128 + 4 * fq, efq = fq;
        asm volatile("" : "+v"(erow), "+v"(ecol), "+v"(efq));
        if constexpr (E == Epi::Int32) {
            issue_after_epilogue_reads(g);
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
                const int mr = m0 + wm * 64 + 16 * bj;            // first row of the block (uniform)
                const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
                    static_cast<int32_t *>(p.y) + (int64_t)mr * p.N, (short)0, NUM_RECORDS, 0x00020000);
                const bool rok = mr + erow < Mi;
#pragma unroll
                for (int bi = 0; bi < 8; ++bi) {
                    const int n = n0 + ecol + 16 * bi;
                    const v4u d = {(unsigned)acc[bi][bj][0], (unsigned)acc[bi][bj][1], (unsigned)acc[bi][bj][2],
                                   (unsigned)acc[bi][bj][3]};
                    if constexpr (VEC) {
                        const uint32_t off = (rok && n < Ni) ? (uint32_t)(erow * Ni + n) * 4u : OOB;
                        __builtin_amdgcn_raw_buffer_store_b128(d, ry, off, 0, 0);
                    } else {
                        // rows not 16-byte aligned (N % 8 != 0): element stores, clipped at N
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
            issue_after_epilogue_reads(g);
            int32_t *slot = p.part + (int64_t)J.slot * (BM * BN);
            // own laundered lane bases, so that no address of this branch is shared with (and kept
            // live across) the bf16 branch
            int prow = frow, pcol = wn * 128 + 4 * fq;
            asm volatile("" : "+v"(prow), "+v"(pcol));
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
                const int ml = wm * 64 + 16 * bj;
                const __amdgpu_buffer_rsrc_t rp =
                    __builtin_amdgcn_make_buffer_rsrc(slot + ml * BN, (short)0, NUM_RECORDS, 0x00020000);
                const bool rok = m0 + ml + prow < Mi;
#pragma unroll
                for (int bi = 0; bi < 8; ++bi) {
                    const int nl = pcol + 16 * bi;
                    const v4u d = {(unsigned)acc[bi][bj][0], (unsigned)acc[bi][bj][1], (unsigned)acc[bi][bj][2],
                                   (unsigned)acc[bi][bj][3]};
                    const uint32_t off = (rok && n0 + nl < Ni) ? (uint32_t)(prow * BN + nl) * 4u : OOB;
                    __builtin_amdgcn_raw_buffer_store_b128(d, rp, off, 0, 0);
                }
                fence();
            }
        } else if constexpr (VEC) {
            const float *ls = reinterpret_cast<const float *>(smem + SCALE_OFF + (j & (NSCALE - 1)) * SCALE_BYTES);
            // the wave's region: piece q (0..7) at 1024 w + 8192 (q & 3) (+ OPB for q >= 4); row r
            // of a 32-row block is piece r / 4 at (r % 4) * 256, its 16-byte chunk c at position
            // c ^ (r % 16).  A lane writes its 4 columns (8 bytes) of a 16x16 block as one half of
            // a chunk: the 16 lanes of a column group cover 16 rows whose chunk positions differ,
            // and the next 16 lanes the other halves, so each 32-lane write fills all 64 banks.
            uint8_t *reg = smem + (g & (NST - 1)) * STAGE + w * 1024;
            // lane-dependent parts, laundered so that they are formed here rather than hoisted
            // out of the tile loop (where they would stay live, or spill):
            //   write side: row erow's base in the region (rows erow and erow + 16 of the 32-row
            //               block: + OPB), the XOR key of its chunk positions, and the lane's half
            //               chunk: columns 4 fq .. 4 fq + 3 of a 16-column block are chunk
            //               2 bi + fq / 2 of the row, half fq % 2
            //   read side:  instruction q reads row r = 4q + rrow, chunk rchunk, at position
            //               rchunk ^ (r % 16) = (rchunk ^ rrow) ^ 4 (q % 4)
            int wrow = 8192 * ((erow >> 2) & 3) + (erow & 3) * 256 + 8 * (efq & 1), wkey = (efq >> 1) ^ erow;
            int rrow = lane >> 4, rchunk = lane & 15, rkey = rchunk ^ (lane >> 4);
            asm volatile("" : "+v"(wrow), "+v"(wkey), "+v"(rrow), "+v"(rchunk), "+v"(rkey));
            const int n = n0 + wn * 128 + 8 * rchunk;
#pragma unroll
            for (int bp = 0; bp < 2; ++bp) {
#pragma unroll
                for (int b2 = 0; b2 < 2; ++b2) {
                    const int bj = 2 * bp + b2;
                    const float sxm = ls[2 * BN + wm * 64 + 16 * bj + erow];
#pragma unroll
                    for (int bi = 0; bi < 8; ++bi) {
                        const int nl = ecol + 16 * bi;
                        const v4f s4 = *reinterpret_cast<const v4f *>(ls + nl);
                        const v4f b4 = *reinterpret_cast<const v4f *>(ls + BN + nl);
                        float yv[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) yv[i] = __builtin_fmaf((float)acc[bi][bj][i], sxm * s4[i], b4[i]);
                        // chunk 2 bi + fq / 2 of row erow + 16 b2, at position chunk ^ (erow % 16)
                        *reinterpret_cast<v2u *>(reg + b2 * OPB + wrow + 16 * ((2 * bi) ^ wkey)) =
                            v2u{pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3])};
                    }
                }
                // back in row order: instruction q reads rows 4q .. 4q+3, 16 lanes per row
                v4u out[8];
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    out[q] = *reinterpret_cast<const v4u *>(reg + (q >> 2) * OPB + 8192 * (q & 3) + rrow * 256 +
                                                            16 * (rkey ^ (4 * (q & 3))));
                // the loads of K-tile g + 2 refill the region: after the last block's reads, before
                // its stores (the first barrier of the next job then waits for all but those 8)
                if (bp == 1) issue_after_epilogue_reads(g);
                const int mr = m0 + wm * 64 + 32 * bp;
                const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
                    static_cast<uint16_t *>(p.y) + (int64_t)mr * p.N, (short)0, NUM_RECORDS, 0x00020000);
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int r = 4 * q + rrow;
                    const uint32_t off = (mr + r < Mi && n < Ni) ? (uint32_t)(r * Ni + n) * 2u : OOB;
                    __builtin_amdgcn_raw_buffer_store_b128(out[q], ry, off, 0, 0);
                }
                fence();
            }
        } else {
            issue_after_epilogue_reads(g);
            const float *ls = reinterpret_cast<const float *>(smem + SCALE_OFF + (j & (NSCALE - 1)) * SCALE_BYTES);
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
                const int mr = m0 + wm * 64 + 16 * bj;
                const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
                    static_cast<uint16_t *>(p.y) + (int64_t)mr * p.N, (short)0, NUM_RECORDS, 0x00020000);
                const bool rok = mr + erow < Mi;
                const float sxm = ls[2 * BN + wm * 64 + 16 * bj + erow];
#pragma unroll
                for (int bi = 0; bi < 8; ++bi) {
                    const int nl = ecol + 16 * bi;
                    const v4f s4 = *reinterpret_cast<const v4f *>(ls + nl);
                    const v4f b4 = *reinterpret_cast<const v4f *>(ls + BN + nl);
                    const int n = n0 + nl;
                    // rows not 16-byte aligned (N % 8 != 0): element stores, clipped at N
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float yv = __builtin_fmaf((float)acc[bi][bj][e], sxm * s4[e], b4[e]);
                        const uint32_t off = (rok && n + e < Ni) ? (uint32_t)(erow * Ni + n + e) * 2u : OOB;
                        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(pack_bf16x2(yv, 0.0f) & 0xffffu), ry, off,
                                                              0, 0);
                    }
                }
                fence();
            }
        }
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = v4i{};
    };

    if (njobs <= 0) return;
    // Stores each wavefront issues after the loads of the next job's second K-tile, in an
    // epilogue (vmcnt counts them too; the int32 and split-unit epilogues issue all 32 of theirs
    // after those loads; the bf16 one 8 of its 16).
    constexpr int EPI_STORES = E == Epi::Int32 ? 32 : 8;
    // Instruction interleaving inside one sub-step's scheduling region (sched_group_barrier masks:
    // 0x008 MFMA, 0x100 LDS read, 0x020 global read): the matrix pipe keeps its queue while the
    // fragment reads and the global loads go out between its instructions.
    // A sub-step has 16 MFMAs and issues 4 or 8 fragment reads, one after each of its first MFMAs.
    auto interleave_reads = [](auto nreads) {
#pragma unroll
        for (int q = 0; q < decltype(nreads)::value; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 16 - decltype(nreads)::value, 0);
    };
    // prologue: K-tile 0 (and job 0's scales) visible, K-tile 1 in flight, first fragments
    next_job();
    issue_ktile(0, true);
    if (ld_kt == ld_ke) next_job();
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();
    issue_ktile(1, true);
    if (ld_kt == ld_ke) next_job();
    read_a(0, 0, 0);
    read_b(0, 0);

    int g = 0;
    for (int j = 0; j < njobs; ++j) {
        // only the K-tile count of the job stays live through its K loop; the epilogue recomputes
        // the rest (scalar registers are scarce here)
        int nkt, first = 1;
        {
            const Job J = job(j);
            nkt = __builtin_amdgcn_readfirstlane(J.ke - J.kb);
        }
        for (int kt = 0; kt < nkt; ++kt, ++g, first = 0) {
            // sub-steps (0,0), (0,1), (1,0): MFMAs on the fragments read one sub-step earlier, the
            // next sub-step's fragments read between them
            read_a(g, 0, 1);
            mfma_range(0, 0, 0, 16);
            interleave_reads(std::integral_constant<int, 4>{});
            fence();
            read_a(g, 1, 0);
            read_b(g, 1);
            mfma_range(0, 1, 0, 16);
            interleave_reads(std::integral_constant<int, 8>{});
            fence();
            read_a(g, 1, 1);
            mfma_range(1, 0, 0, 16);
            interleave_reads(std::integral_constant<int, 4>{});
            fence();
            // sub-step (1,1) starts before the barrier: these MFMAs use registers only, and keep the
            // matrix pipe busy while the wavefronts meet
            mfma_range(1, 1, 0, 4);
            fence();
            // K-tile g+1 must have landed before its first fragments are read: at most the
            // previous tile's epilogue stores may still be in flight right after an epilogue (and
            // only with 16-byte stores; otherwise wait for everything).
            if (VEC && j > 0 && first) __builtin_amdgcn_s_waitcnt(waitcnt_vm(EPI_STORES));
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            // Every wave has completed (lgkmcnt(0)) its reads of stage g & 1 and waited for its
            // loads of K-tile g+1.  A raw barrier: the fence of __syncthreads() would make the
            // compiler wait for every store in flight as well.
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            // rest of sub-step (1,1): the loads of K-tile g+2 into the stage just freed and the first
            // fragments of K-tile g+1 go out between the MFMAs (past the end of the stream the
            // loads are out of range and the reads of a stale stage are never used).  After a
            // job's last K-tile the epilogue uses the freed stage first and issues the loads itself.
            issue_ktile(g, kt + 1 < nkt);
            read_a(g + 1, 0, 0);
            read_b(g + 1, 0);
            mfma_range(1, 1, 4, 16);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            }
            fence();
            if (ld_kt == ld_ke) next_job();
            fence();
        }
        epilogue(job(j), j, g - 1);
    }
    // the stream's last (out-of-range) loads write zeros into LDS: let them land before the
    // workgroup's LDS is released
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
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
    p.M = (int)M;
    p.N = (int)N;
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
    // 16-byte stores of 4 (int32) or 8 (bf16) columns need N % 8 == 0; otherwise element stores
    if (epi == Epi::Int32 && N % 8 == 0)
        hipLaunchKernelGGL((gemm_i8_kernel<Epi::Int32, true>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream, p);
    else if (epi == Epi::Int32)
        hipLaunchKernelGGL((gemm_i8_kernel<Epi::Int32, false>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream, p);
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
