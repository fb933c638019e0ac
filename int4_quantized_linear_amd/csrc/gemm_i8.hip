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
//  * workgroup tile 256(M) x 256(N), 4 wavefronts in 2x2, each owning a 128x128 sub-tile as
//    4x4 blocks of v_mfma_i32_32x32x32_i8 (256 int32 accumulators per lane);
//  * K is staged 128 bytes at a time through a double-buffered LDS (2 x 64 KiB) with
//    buffer_load ... lds (global -> LDS without VGPRs).  Rows are stored with their 16-byte
//    chunks XOR-swizzled by (row & 7) so the ds_read_b128 fragment reads are conflict-free;
//    each load instruction still reads whole 128-byte lines.  Out-of-range rows and K chunks
//    are read through an out-of-bounds buffer offset, which returns zeros;
//  * blockIdx -> tile mapping gives each of the 8 XCDs a contiguous run of tiles, walked in
//    groups along M so concurrently running tiles share their weight tile in that XCD's L2;
//  * the epilogue stages the bf16 tile through LDS (padded rows) and writes Y with fully
//    coalesced 16-byte stores.
#include "device_common.hpp"
#include "launchers.hpp"

namespace convrot {
namespace {

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int OPB = 256 * BK;                // bytes of one operand tile per stage (32 KiB)
constexpr int STAGE = 2 * OPB;               // W tile then X tile
constexpr int EPI_PITCH = BN * 2 + 16;       // bytes per staged bf16 output row
constexpr int SMEM = (2 * STAGE > BM * EPI_PITCH) ? 2 * STAGE : BM * EPI_PITCH;
constexpr int GROUP_M = 16;
constexpr uint32_t OOB = 0x80000000u;        // buffer offset past num_records -> loads return 0
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
};

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= n only.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }

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

template <Epi E>
__global__ void __launch_bounds__(256, 1) gemm_i8_kernel(GemmParams p)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int wn = w & 1, wm = w >> 1;
    int tm, tn;
    tile_of(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int K = p.K;

    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(p.wq + n0 * K), (short)0, NUM_RECORDS, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(p.xq + m0 * K), (short)0, NUM_RECORDS, 0x00020000);

    // This lane's 16-byte chunk of each of the 8 load instructions per operand and stage:
    // instruction i of wave w fills LDS rows 8*(4i+w) .. +7; lane -> row +lane/8, swizzled
    // position lane%8, i.e. K chunk (lane%8) ^ (lane/8).
    const int lchunk = (lane & 7) ^ (lane >> 3);
    uint32_t offw[8], offx[8];
    bool okw[8], okx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = 8 * (4 * i + w) + (lane >> 3);
        okw[i] = n0 + row < p.N;
        okx[i] = m0 + row < p.M;
        offw[i] = (uint32_t)(row * K + 16 * lchunk);
        offx[i] = offw[i];
    }

    auto issue = [&](int kt, int stage) {
        const int k0 = kt * BK;
        const bool kok = k0 + 16 * lchunk < K;
        uint8_t *base = smem + stage * STAGE;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t ow = (okw[i] && kok) ? offw[i] + k0 : OOB;
            const uint32_t ox = (okx[i] && kok) ? offx[i] + k0 : OOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(base + (4 * i + w) * 1024), 16, ow, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(base + OPB + (4 * i + w) * 1024), 16, ox, 0, 0, 0);
        }
    };

    v16i acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = v16i{};

    // Fragment addressing: row = wave base + 32*blk + lane%32 (so row & 7 == lane & 7) and
    // K chunk = 2*kk + lane/32 of the 8 chunks of a 128-byte stage row.
    const int frow = lane & 31, fhalf = lane >> 5, fsw = lane & 7;
    const int arow = (wn * 128 + frow) * BK, brow = OPB + (wm * 128 + frow) * BK;
    v4i fa[2][4], fb[2][4];
    auto read_frags = [&](int stage, int kk, int buf) {
        const uint8_t *s0 = smem + stage * STAGE;
        const int pos = ((2 * kk + fhalf) ^ fsw) * 16;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            fa[buf][b] = *reinterpret_cast<const v4i *>(s0 + arow + 32 * b * BK + pos);
            fb[buf][b] = *reinterpret_cast<const v4i *>(s0 + brow + 32 * b * BK + pos);
        }
    };
    auto mfmas = [&](int buf) {
#pragma unroll
        for (int bi = 0; bi < 4; ++bi)
#pragma unroll
            for (int bj = 0; bj < 4; ++bj)
                acc[bi][bj] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[buf][bi], fb[buf][bj], acc[bi][bj], 0, 0, 0);
    };

    // Pipeline: LDS holds tiles t (being read) and t+1 (landing).  Each tile's last fragments
    // are read into registers before the barrier, so right after it the stage of tile t is
    // refilled with tile t+2 and tile t+1's first fragments are read while the last 16 MFMAs
    // of tile t run.
    const int KT = (K + BK - 1) / BK;
    issue(0, 0);
    if (KT > 1) {
        issue(1, 1);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(16));   // tile 0 landed, tile 1 in flight
    } else {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    __syncthreads();
    read_frags(0, 0, 0);

    for (int kt = 0; kt < KT; ++kt) {
        const int stage = kt & 1;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            if (kk < 3) {
                read_frags(stage, kk + 1, (kk + 1) & 1);
            } else {
                __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0): tile t+1 landed, tile t read
                __syncthreads();
                if (kt + 2 < KT) issue(kt + 2, stage);
                if (kt + 1 < KT) read_frags(stage ^ 1, 0, 0);
            }
            mfmas(kk & 1);
        }
    }

    // Accumulator layout of a 32x32 block (MFMA rows = weight rows n, columns = tokens m):
    // lane holds m = lane%32 and, for register v, n = 8*(v/4) + 4*(lane/32) + v%4.
    if constexpr (E == Epi::Int32) {
        int32_t *y = static_cast<int32_t *>(p.y);
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            const int64_t m = m0 + wm * 128 + 32 * bj + frow;
            if (m >= p.M) continue;
#pragma unroll
            for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t n = n0 + wn * 128 + 32 * bi + 8 * g + 4 * fhalf + i;
                        if (n < p.N) y[m * p.N + n] = acc[bi][bj][4 * g + i];
                    }
        }
    } else {
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            const int ml = wm * 128 + 32 * bj + frow;
            const int64_t m = m0 + ml;
            const float sxm = m < p.M ? p.sx[m] : 0.0f;
#pragma unroll
            for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int nl = wn * 128 + 32 * bi + 8 * g + 4 * fhalf;
                    float yv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t n = n0 + nl + i;
                        const float swn = n < p.N ? p.sw[n] : 0.0f;
                        const float bn = (p.bias && n < p.N) ? p.bias[n] : 0.0f;
                        yv[i] = __builtin_fmaf((float)acc[bi][bj][4 * g + i], sxm * swn, bn);
                    }
                    uint2 pk;
                    pk.x = pack_bf16x2(yv[0], yv[1]);
                    pk.y = pack_bf16x2(yv[2], yv[3]);
                    *reinterpret_cast<uint2 *>(smem + ml * EPI_PITCH + nl * 2) = pk;
                }
        }
        __syncthreads();
        uint16_t *y = static_cast<uint16_t *>(p.y);
        const int ch = threadIdx.x & 31;
        const bool vec = (p.N & 7) == 0;
        for (int rp = 0; rp < BM; rp += 8) {
            const int row = rp + (threadIdx.x >> 5);
            const int64_t m = m0 + row;
            const int64_t n = n0 + 8 * ch;
            if (m >= p.M || n >= p.N) continue;
            const uint4 v = *reinterpret_cast<const uint4 *>(smem + row * EPI_PITCH + 16 * ch);
            if (vec) {
                *reinterpret_cast<uint4 *>(y + m * p.N + n) = v;
            } else {
                const uint16_t *e = reinterpret_cast<const uint16_t *>(&v);
                for (int i = 0; i < 8 && n + i < p.N; ++i) y[m * p.N + n + i] = e[i];
            }
        }
    }
}

} // namespace

hipError_t launch_gemm_i8(const int8_t *xq, const int8_t *wq, const float *sx, const float *sw, const float *bias,
                          void *y, Epi epi, int64_t M, int64_t N, int K, hipStream_t stream)
{
    if (M <= 0 || N <= 0) return hipSuccess;
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
    p.tiles_m = (int)((M + BM - 1) / BM);
    p.tiles_n = (int)((N + BN - 1) / BN);
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(256);
    if (epi == Epi::Int32)
        hipLaunchKernelGGL(gemm_i8_kernel<Epi::Int32>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(gemm_i8_kernel<Epi::Bf16>, grid, block, 0, stream, p);
    return hipGetLastError();
}

} // namespace convrot
