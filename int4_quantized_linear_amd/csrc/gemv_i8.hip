// gemv_i8.hip -- decode-shaped ConvRot linear (M <= 16 tokens), weight-bandwidth bound (gfx950).
//
// Same contraction and epilogue as the GEMM (acc = xq . wq^T, y = bf16(acc*sx*sw + bias)), for
// the few-token case: the conditioning pass of the text encoder on the pages runs at 12 tokens
// ("Qwen3-VL-32B-...-INT8-ConvRot部署优化", section 运行时验证指标, output (1, 12, 5120)), so every
// ConvRot linear there streams its whole INT8 weight once for 12 rows of work.
//
// Design: a workgroup owns RB 16-row blocks of weights (16, 32 or 64 rows) and all of K; its NW
// wavefronts split K into contiguous runs of 256-byte chunks.  Each wavefront streams its run on
// its own, with no barrier in the main loop: per chunk it copies its rows' 256 bytes and the
// <= 16 token rows' 256 bytes global -> LDS (buffer_load ... lds, 16 bytes per lane; one
// instruction moves 4 rows x 256 contiguous bytes, i.e. whole 128-byte lines) into a private
// ring of D stages, and waits for them with its own vmcnt.  In a stage, 16-byte chunk c of row
// r sits at position c ^ (r & 15), so the MFMA fragment reads (16 rows, same chunk) hit 16
// distinct bank groups.  Rows >= N, tokens >= M and bytes past K read zeros through
// out-of-bounds buffer offsets.  v_mfma_i32_16x16x64_i8 (rows = weight rows, columns = tokens)
// accumulates the whole run in int32 (|acc| <= 127^2 K < 2^31 for K <= 131072); the NW sums
// are added once at the end through LDS (exact in any order) and the epilogue writes bf16 (or
// the int32 sums).  There is no cross-workgroup split of K: joining partial sums across CUs
// needs several trips to the device-coherent level, about a microsecond each, which is more
// than a small decode call costs in total; small N gets more wavefronts per workgroup instead.
#include "device_common.hpp"
#include "launchers.hpp"

namespace convrot {
namespace {

constexpr int KC = 256;                  // K bytes per row per chunk (4 MFMA K-steps)
constexpr int D = 2;                     // LDS stages per wavefront
constexpr int MAX_NW = 8;
constexpr int TARGET_WAVES = 400;        // about 1.5 wavefronts per CU in all
constexpr int MIN_CHUNKS = 5;            // per wavefront, to amortise its ramp-up and drain
constexpr int LDS_BUDGET = 160 * 1024;
constexpr uint32_t OOB = 0x80000000u;    // buffer offset past num_records -> loads return 0
constexpr int NUM_RECORDS = 0x7ffffff0;

typedef __attribute__((address_space(3))) void lds_void;

struct GemvParams {
    const int8_t *xq;
    const int8_t *wq;
    const float *sx;
    const float *sw;
    const float *bias;
    void *y;
    int64_t N;
    int M, K;
};

// s_waitcnt immediate waiting for vmcnt <= n only (gfx9 encoding)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }

template <int RB>
constexpr int stage_bytes() { return (16 * RB + 16) * KC; }   // weight rows + 16 token rows

// Copies of one chunk into a stage: copy j moves rows 4j + lane/16 of the stage (weight rows,
// then the 16 token rows); lane%16 is the 16-byte position, holding chunk (lane%16) ^ (row & 15).
// Offsets come precomputed per copy (row start + swizzled position, bit 31 set for rows past N or
// tokens past M); here they get the chunk's K position, and bit 31 for pieces past K or for a
// chunk past the run (out of range: zeros, no memory access).  Plain arithmetic rather than
// selects, which the compiler would turn into branches around the loads.
template <int RB>
__device__ __forceinline__ void copy_chunk(uint8_t *st, __amdgpu_buffer_rsrc_t rw, __amdgpu_buffer_rsrc_t rx,
                                           const uint32_t *wrow, const uint32_t *xrow, int k0, uint32_t dead, int K,
                                           int cr, int px)
{
#pragma unroll
    for (int j = 0; j < 4 * RB; ++j) {
        const int rr = 4 * j + cr;
        const uint32_t past = (uint32_t)(k0 + 16 * (px ^ (rr & 15)) >= K) << 31;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(st + 1024 * j), 16,
                                                 (wrow[j] + (uint32_t)k0) | dead | past, 0, 0, 2);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = 4 * j + cr;
        const uint32_t past = (uint32_t)(k0 + 16 * (px ^ t) >= K) << 31;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(st + 16 * RB * KC + 1024 * j), 16,
                                                 (xrow[j] + (uint32_t)k0) | dead | past, 0, 0, 0);
    }
}

template <Epi E, int RB>
__global__ void __launch_bounds__(64 * MAX_NW) gemv_i8_kernel(GemvParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int WL = 4 * RB;                           // weight copies per chunk (4 rows each)
    constexpr int LPC = WL + 4;                          // + 4 token copies
    constexpr int STAGE = stage_bytes<RB>();
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * (16 * RB);
    const int K = p.K;
    const int C = (K + KC - 1) / KC;
    const int c_beg = C * w / nw;                        // nw <= C: every run has a chunk
    const int c_end = C * (w + 1) / nw;
    const int n = c_end - c_beg;
    const int r = lane & 15, q = lane >> 4;
    const int M = p.M;
    const int m = r;

    // epilogue operands first, so that their latency hides under the main loop
    float coef[RB][4], bia[RB][4];
    if (E == Epi::Bf16 && w == 0) {
        const float sxm = p.sx[m < M ? m : 0];
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t nn = n0 + 16 * b + 4 * q + v;
                const int64_t nc = nn < p.N ? nn : 0;
                coef[b][v] = sxm * p.sw[nc];
                bia[b][v] = p.bias ? p.bias[nc] : 0.0f;
            }
    }

    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t *>(p.wq + n0 * K), (short)0, NUM_RECORDS, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(p.xq), (short)0, NUM_RECORDS, 0x00020000);
    uint8_t *ring = smem + w * (D * STAGE);
    const int cr = lane >> 4, px = lane & 15;
    uint32_t wrow[WL], xrow[4];
#pragma unroll
    for (int j = 0; j < WL; ++j) {
        const int rr = 4 * j + cr;
        wrow[j] = ((uint32_t)(rr * K + 16 * (px ^ (rr & 15)))) | ((uint32_t)(n0 + rr >= p.N) << 31);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int t = 4 * j + cr;
        xrow[j] = ((uint32_t)(t * K + 16 * (px ^ t))) | ((uint32_t)(t >= M) << 31);
    }
    // chunk c of this wavefront = K bytes [256 (c_beg + c), +256)
    auto load = [&](int slot, int c) {
        copy_chunk<RB>(ring + slot * STAGE, rw, rx, wrow, xrow, (c_beg + c) * KC, (uint32_t)(c >= n) << 31, K, cr, px);
    };

    v4i acc[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) acc[b] = v4i{};

    auto compute = [&](int slot) {
        // this chunk has landed once at most the next chunk's copies remain in flight
        __builtin_amdgcn_s_waitcnt(waitcnt_vm((D - 1) * LPC));
        const uint8_t *st = ring + slot * STAGE;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int pos = 16 * ((4 * kk + q) ^ r);
            const v4i xb = *reinterpret_cast<const v4i *>(st + 16 * RB * KC + r * KC + pos);
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                const v4i a = *reinterpret_cast<const v4i *>(st + (16 * b + r) * KC + pos);
                acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, xb, acc[b], 0, 0, 0);
            }
        }
    };

#pragma unroll
    for (int j = 0; j < D; ++j) {
        load(j, j);
        __builtin_amdgcn_sched_barrier(0);
    }
    // whole rounds of D chunks, so that the loop body has no branch (a join would make the
    // compiler drain every load in flight); chunks past the run are zeros and add nothing
    for (int c0 = 0; c0 < n; c0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            compute(j);
            // the fragment reads of this stage must finish before its refill lands
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            load(j, c0 + j + D);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    if (nw > 1) {
        __syncthreads();                                 // every ring is idle: reuse the LDS
        int32_t *red = reinterpret_cast<int32_t *>(smem);   // [nw][RB * 4][64]
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[(w * RB * 4 + 4 * b + v) * 64 + lane] = acc[b][v];
        __syncthreads();
        if (w != 0) return;
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                int32_t s = red[(4 * b + v) * 64 + lane];
                for (int ww = 1; ww < nw; ++ww) s += red[(ww * RB * 4 + 4 * b + v) * 64 + lane];
                acc[b][v] = s;
            }
    }
    if (m >= M) return;
    // 16x16 layout: lane holds token m = lane%16 and rows 4*(lane/16) + v of each 16-row block
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t nn = n0 + 16 * b + 4 * q + v;
            if (nn >= p.N) continue;
            if constexpr (E == Epi::Int32) {
                static_cast<int32_t *>(p.y)[(int64_t)m * p.N + nn] = acc[b][v];
            } else {
                const float yv = __builtin_fmaf((float)acc[b][v], coef[b][v], bia[b][v]);
                static_cast<uint16_t *>(p.y)[(int64_t)m * p.N + nn] = (uint16_t)(pack_bf16x2(yv, 0.0f) & 0xffffu);
            }
        }
}

struct Plan {
    int rb, nw;
    int64_t tiles;
};

// Rows per workgroup: 64 from N = 16384 on, 32 from N = 4096, else 16 (more workgroups for small
// N; each one re-reads the tokens).  Wavefronts per workgroup: about TARGET_WAVES in all, each
// with at least MIN_CHUNKS chunks, within the LDS budget (D stages per wavefront).  Both
// measured on the decode shapes (N x K = 8192/1024/25600 x 5120, 5120 x 25600): fewer,
// longer-running wavefronts beat many short ones.
Plan plan(int64_t N, int K)
{
    Plan pl;
    pl.rb = N >= 16384 ? 4 : N >= 4096 ? 2 : 1;
    pl.tiles = (N + 16 * pl.rb - 1) / (16 * pl.rb);
    const int C = (K + KC - 1) / KC;
    int64_t nw = (TARGET_WAVES + pl.tiles - 1) / pl.tiles;
    if (nw > C / MIN_CHUNKS) nw = C / MIN_CHUNKS;
    const int per_wave = D * (pl.rb == 4 ? stage_bytes<4>() : pl.rb == 2 ? stage_bytes<2>() : stage_bytes<1>());
    if (nw > LDS_BUDGET / per_wave) nw = LDS_BUDGET / per_wave;
    if (nw > MAX_NW) nw = MAX_NW;
    pl.nw = nw < 1 ? 1 : (int)nw;
    return pl;
}

} // namespace

hipError_t launch_gemv_i8(const int8_t *xq, const int8_t *wq, const float *sx, const float *sw, const float *bias,
                          void *y, Epi epi, int64_t M, int64_t N, int K, hipStream_t stream)
{
    if (M <= 0 || N <= 0) return hipSuccess;
    GemvParams p;
    p.xq = xq;
    p.wq = wq;
    p.sx = sx;
    p.sw = sw;
    p.bias = bias;
    p.y = y;
    p.N = N;
    p.M = (int)M;
    p.K = K;
    const Plan pl = plan(N, K);
    const dim3 grid((unsigned)pl.tiles), block(64 * pl.nw);
    const size_t lds =
        (size_t)pl.nw * D * (pl.rb == 4 ? stage_bytes<4>() : pl.rb == 2 ? stage_bytes<2>() : stage_bytes<1>());
    if (epi == Epi::Int32) {
        if (pl.rb == 4)
            hipLaunchKernelGGL((gemv_i8_kernel<Epi::Int32, 4>), grid, block, lds, stream, p);
        else if (pl.rb == 2)
            hipLaunchKernelGGL((gemv_i8_kernel<Epi::Int32, 2>), grid, block, lds, stream, p);
        else
            hipLaunchKernelGGL((gemv_i8_kernel<Epi::Int32, 1>), grid, block, lds, stream, p);
    } else {
        if (pl.rb == 4)
            hipLaunchKernelGGL((gemv_i8_kernel<Epi::Bf16, 4>), grid, block, lds, stream, p);
        else if (pl.rb == 2)
            hipLaunchKernelGGL((gemv_i8_kernel<Epi::Bf16, 2>), grid, block, lds, stream, p);
        else
            hipLaunchKernelGGL((gemv_i8_kernel<Epi::Bf16, 1>), grid, block, lds, stream, p);
    }
    return hipGetLastError();
}

} // namespace convrot
