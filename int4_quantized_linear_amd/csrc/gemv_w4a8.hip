// gemv_w4a8.hip -- decode-shaped W4A8 ConvRot linear (M <= 16 tokens), weight-bandwidth bound.
//
// INT4 weights (one fp16 scale per (row, 256-channel group)) against INT8 tokens (one fp32 scale
// per token), both rotated by the same grouped Hadamard (the W4A8 format of the MiniMax-H3
// W4A8 ConvRot pages: 4-bit weights, 8-bit activations):
//   y[m,n] = bf16( sx[m] * sum_j sw[j,n] * (sum_{k in group j} qx[m,k] * cw[n,k]) + bias[n] )
//
// Weights are re-laid out once (pack_w4a8_kernel) into the order the kernel consumes them, so
// every load instruction of the hot loop reads 1 KiB of contiguous memory:
//   tile t (64 rows) x group j -> one block of BS = 8320 bytes at (t * G + j) * BS:
//     codes: 8 pieces of 1 KiB, piece (b, i) = row block b (rows 16b..16b+15), half i;
//            lane l = (r = l % 16, q = l / 16) owns 16 bytes = K-steps 2i and 2i+1 of row
//            16b + r, each K-step two dwords (dA, dB) over the 16 channels
//            k = 64 kk + 16 q + s (s = 0..15) of the group: byte u of dA holds channel s = u in
//            its high nibble and s = 4 + u in its low nibble, dB the same for s = 8+u, 12+u;
//     scales: 128 bytes, fp16 of row 16b + 4q + v at byte 32q + 8b + 2v (zero for rows >= N).
//   Rows past N are zero codes with zero scales.
// With that nibble order one K-step's MFMA operand is
//   [dA & 0xF0F0F0F0, (dA << 4) & 0xF0F0F0F0, dB & 0xF0F0F0F0, (dB << 4) & 0xF0F0F0F0]
// = the 16 codes times 16 as int8 in channel order (3 VALU per packed dword).
//
// GEMV: a workgroup owns 16 or 32 rows (one or two 16-row blocks of a packed tile) and all of K;
// its NW wavefronts split K into contiguous runs of whole groups.  Each wavefront streams its run
// on its own, with no barrier in the main loop: per group it loads its code pieces and scale
// bytes into a ring of D chunks in registers and the group's 16 token rows into its own LDS ring
// (load-to-LDS, 1 KiB per instruction; token t keeps 16-byte chunk c at c ^ t, so the fragment
// reads are conflict-free; tokens >= M arrive as zeros).  Per group it computes the 16x16 blocks
// with v_mfma_i32_16x16x64_i8 (rows = weights, columns = tokens) and folds them:
// facc += float(iacc) * sw (iacc is 16x the integer dot product, exact in fp32; the 1/16 goes
// into the final token scale).  The NW partial results are added once at the end through LDS in
// wavefront order (deterministic).  There is no cross-workgroup reduction: that needs several
// trips to the device-coherent level, about a microsecond each, more than a small decode call
// costs in total.  Small N therefore gets more wavefronts per workgroup rather than split-K
// workgroups (see plan()).
#include "device_common.hpp"
#include "launchers.hpp"

namespace convrot {
namespace {

constexpr int GS = 256;                  // channels per scale group
constexpr int RBW = 4;                   // 16-row blocks per tile
constexpr int RT = 16 * RBW;             // rows per tile
constexpr int CODE_BYTES = RT * GS / 2;  // 8 KiB
constexpr int BS = CODE_BYTES + 2 * RT;  // + the tile's 64 fp16 scales
// 128-channel scale groups (the dynamic group of a width 256 does not divide): a block keeps
// 256 channels and carries two scale sets, half i's at CODE_BYTES + 128 i (the pieces (b, i)
// are exactly channels 128 i .. 128 i + 127 of the block); when K % 256 == 128 the last block's
// upper half is zero codes with zero scales.
constexpr int BS128 = CODE_BYTES + 4 * RT;
template <bool G128>
constexpr int block_bytes() { return G128 ? BS128 : BS; }
constexpr int TARGET_WAVES = 640;       // about 2.5 wavefronts per CU in all
constexpr int MIN_GROUPS = 5;            // per wavefront, to amortise its ramp-up and drain
constexpr uint32_t OOB = 0x80000000u;
constexpr int NUM_RECORDS = 0x7ffffff0;

typedef __attribute__((address_space(3))) void lds_void;

// ------------------------------------------------------------------ packing

// One thread per 16-byte code piece or per 8-byte scale quad of a block.
template <bool G128>
__global__ void __launch_bounds__(256) pack_w4a8_kernel(const uint8_t *__restrict__ wq, const uint16_t *__restrict__ sw,
                                                        uint8_t *__restrict__ out, int64_t N, int K, int64_t nblocks)
{
    const int G = (K + GS - 1) / GS;
    const int Kh = K / 2;
    constexpr int NSC = G128 ? 2 : 1;                    // scale sets per block
    const int per_block = CODE_BYTES / 16 + NSC * RT / 4;   // 512 pieces + 16 scale quads per set
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= nblocks * per_block) return;
    const int64_t blk = idx / per_block;
    const int piece = (int)(idx % per_block);
    const int64_t t = blk / G;
    const int j = (int)(blk % G);
    uint8_t *dst = out + blk * block_bytes<G128>();
    if (piece < CODE_BYTES / 16) {
        const int bi = piece >> 6, l = piece & 63;
        const int b = bi >> 1, i = bi & 1;
        const int r = l & 15, q = l >> 4;
        const int64_t row = t * RT + 16 * b + r;
        uint32_t d[4] = {0u, 0u, 0u, 0u};
        if (row < N) {
            const uint8_t *src = wq + row * Kh + (int64_t)j * (GS / 2);
            for (int h = 0; h < 2; ++h) {                // K-step kk = 2i + h
                const int kk = 2 * i + h;
                // K % 128 == 0, so a 64-channel K-step lies wholly below K or wholly past it (the
                // zero upper half of the last block when K % 256 == 128): one test per K-step
                // keeps the byte loads below unconditional
                if (j * GS + 64 * kk >= K) continue;
                uint32_t nib[16];
#pragma unroll
                for (int s = 0; s < 16; ++s) {
                    const int k = 64 * kk + 16 * q + s;  // channel within the block
                    const uint8_t byte = src[k >> 1];
                    nib[s] = (k & 1) ? (byte >> 4) : (byte & 15u);
                }
                uint32_t dA = 0, dB = 0;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    dA |= ((nib[u] << 4) | nib[4 + u]) << (8 * u);
                    dB |= ((nib[8 + u] << 4) | nib[12 + u]) << (8 * u);
                }
                d[2 * h] = dA;
                d[2 * h + 1] = dB;
            }
        }
        uint32_t *o = reinterpret_cast<uint32_t *>(dst + 1024 * bi + 16 * l);
        for (int u = 0; u < 4; ++u) o[u] = d[u];
    } else {
        const int sq = piece - CODE_BYTES / 16;          // (set, q, b)
        const int set = sq >> 4, q = (sq >> 2) & 3, b = sq & 3;
        const int gi = NSC * j + set;                    // scale group index
        const bool gok = gi < K / (GS / NSC);
        uint16_t v4[4];
        for (int v = 0; v < 4; ++v) {
            const int64_t row = t * RT + 16 * b + 4 * q + v;
            v4[v] = (row < N && gok) ? sw[(int64_t)gi * N + row] : (uint16_t)0;
        }
        uint16_t *o = reinterpret_cast<uint16_t *>(dst + CODE_BYTES + (2 * RT) * set + 32 * q + 8 * b);
        for (int v = 0; v < 4; ++v) o[v] = v4[v];
    }
}

// ------------------------------------------------------------------ GEMV

struct W4A8Params {
    const int8_t *xq;
    const uint8_t *wp;       // packed blocks
    const float *sx;
    const float *bias;
    uint16_t *y;
    int64_t N;
    int M, K;
};

template <int RB, bool G128>
struct Chunk {
    v4i wa[RB][2];                       // code pieces (b0 + b, i)
    uint32_t sc[G128 ? 2 : 1][2 * RB];   // scale set s: fp16 of rows 16(b0 + b) + 4q + v, half v of dword 2b + v/2
};

__device__ __forceinline__ v4i widen_step(uint32_t dA, uint32_t dB)
{
    v4i o;
    o[0] = (int)(dA & 0xF0F0F0F0u);
    o[1] = (int)((dA << 4) & 0xF0F0F0F0u);
    o[2] = (int)(dB & 0xF0F0F0F0u);
    o[3] = (int)((dB << 4) & 0xF0F0F0F0u);
    return o;
}

// s_waitcnt immediate waiting for vmcnt <= n only (gfx9 encoding)
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }

constexpr int D = 2;                     // chunks (groups) in flight per wavefront
constexpr int XSTAGE = 16 * GS;          // one group of 16 token rows (4 KiB)
constexpr int MAX_NW = 8;                // wavefronts per workgroup

// Workgroup = RB 16-row blocks (rows n0 .. n0 + 16 RB - 1) x all of K; wavefront w takes a
// contiguous run of groups.  Per group it loads its RB code pieces and the scale bytes into a
// register ring and the group's 16 token rows into its own LDS ring (load-to-LDS, 1 KiB per
// instruction, token t keeping 16-byte chunk c at c ^ t; tokens >= M arrive as zeros).
template <int RB, bool G128>
__global__ void __launch_bounds__(64 * MAX_NW) gemv_w4a8_kernel(W4A8Params p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int NSC = G128 ? 2 : 1;
    constexpr int BSZ = block_bytes<G128>();
    constexpr int LPC = 2 * RB + NSC * ((RB + 1) / 2) + 4;   // loads per chunk, token loads last
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = blockDim.x >> 6;
    const int64_t n0 = (int64_t)blockIdx.x * (16 * RB);
    const int64_t t64 = n0 / RT;                         // packed 64-row tile
    const int b0 = (int)(n0 % RT) / 16;                  // first row block inside it
    const int K = p.K;
    const int G = (K + GS - 1) / GS;                     // 256-channel blocks
    const int g_beg = G * w / nw;                        // nw <= G: every run has a block
    const int g_end = G * (w + 1) / nw;
    const int n = g_end - g_beg;
    const int r = lane & 15, q = lane >> 4;
    const int M = p.M;
    const int m = r;

    // epilogue operands first, so that their latency hides under the main loop
    float sxm = 0.0f, bia[RB][4];
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) bia[b][v] = 0.0f;
    if (w == 0) {
        sxm = p.sx[m < M ? m : 0] * 0.0625f;
        if (p.bias) {
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                const int64_t nb = n0 + 16 * b + 4 * q;
#pragma unroll
                for (int v = 0; v < 4; ++v) bia[b][v] = p.bias[nb + v < p.N ? nb + v : 0];
            }
        }
    }

    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t *>(p.wp + t64 * G * (int64_t)BSZ), (short)0, NUM_RECORDS, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(p.xq), (short)0, NUM_RECORDS, 0x00020000);
    uint8_t *xs = smem + w * (D * XSTAGE);               // this wavefront's token ring
    // token load j of a group: tokens 4j + lane/16, position lane%16 holding chunk (lane%16) ^ t
    const int tx = lane >> 4, px = lane & 15;

    // chunk c of this wavefront = group g_beg + c.  Chunks past the run load nothing: bit 31 set
    // in an offset makes it out of range (zeros, no memory access).  Plain arithmetic rather than
    // selects, which the compiler would turn into branches around the loads.
    auto load = [&](Chunk<RB, G128> &ch, int slot, int c) {
        const uint32_t dead = (uint32_t)(c >= n) << 31;
        const int g = g_beg + c;
        const uint32_t blk = (uint32_t)g * (uint32_t)BSZ;
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                ch.wa[b][i] = __builtin_bit_cast(
                    v4i, __builtin_amdgcn_raw_buffer_load_b128(
                             rw, (blk + 1024 * (2 * (b0 + b) + i) + 16 * lane) | dead, 0, 2));
        // this lane's scale bytes [32q + 8 b0, + 8 RB) of each of the block's scale sets (128 bytes each)
#pragma unroll
        for (int st = 0; st < NSC; ++st) {
            const uint32_t so = (blk + CODE_BYTES + 2 * RT * st + 32 * q + 8 * b0) | dead;
            if constexpr (RB == 1) {
                const v2u v = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(rw, so, 0, 0));
                ch.sc[st][0] = v[0];
                ch.sc[st][1] = v[1];
            } else {
#pragma unroll
                for (int h = 0; h < RB / 2; ++h) {
                    const v4u v = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rw, so + 16 * h, 0, 0));
#pragma unroll
                    for (int e = 0; e < 4; ++e) ch.sc[st][4 * h + e] = v[e];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = 4 * j + tx;
            // channels past K (the upper half of the last block when K % 256 == 128) load nothing
            const int kc = g * GS + 16 * (px ^ t);
            const uint32_t off = (uint32_t)(t * K + kc) | dead | ((uint32_t)(t >= M) << 31) | ((uint32_t)(kc >= K) << 31);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(xs + slot * XSTAGE + 1024 * j), 16, off, 0, 0, 0);
        }
    };

    float facc[RB][4];
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) facc[b][v] = 0.0f;

    auto compute = [&](const Chunk<RB, G128> &ch, int slot) {
        // the token rows of this chunk have landed once at most the next chunk's loads remain
        __builtin_amdgcn_s_waitcnt(waitcnt_vm((D - 1) * LPC));
        const uint8_t *xst = xs + slot * XSTAGE + r * GS;
        v4i iacc[RB];
        // fold: facc += float(iacc) * s_w of scale set st, per output
        auto fold = [&](int st) {
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const unsigned short h = (unsigned short)(ch.sc[st][2 * b + (v >> 1)] >> (16 * (v & 1)));
                    facc[b][v] = __builtin_fmaf((float)iacc[b][v], (float)__ushort_as_half(h), facc[b][v]);
                }
        };
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            // token r, chunk 4kk + q of the block (16 channels 64kk + 16q ..)
            const v4i xb = *reinterpret_cast<const v4i *>(xst + 16 * ((4 * kk + q) ^ r));
            const bool first = G128 ? (kk & 1) == 0 : kk == 0;   // a scale group's first K-step
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                const v4i &src = ch.wa[b][kk >> 1];
                const v4i a = widen_step((uint32_t)src[2 * (kk & 1)], (uint32_t)src[2 * (kk & 1) + 1]);
                iacc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, xb, first ? v4i{} : iacc[b], 0, 0, 0);
            }
            if (G128 && kk == 1) fold(0);                // channels 0..127 of the block: scale set 0
        }
        fold(NSC - 1);
    };

    Chunk<RB, G128> ring[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {
        load(ring[j], j, j);
        __builtin_amdgcn_sched_barrier(0);
    }
    // whole rounds of D chunks, so that the loop body has no branch (a join would make the
    // compiler drain every load in flight); chunks past the run are zeros and add nothing
    for (int c0 = 0; c0 < n; c0 += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
            compute(ring[j], j);
            // the ds_reads of this slot must finish before its refill lands
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            load(ring[j], j, c0 + j + D);
            // keep this order: hoisting a later chunk's unpacking here would wait for its loads
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    if (nw > 1) {
        __syncthreads();                                 // every token ring is idle: reuse the LDS
        float *red = reinterpret_cast<float *>(smem);    // [nw][RB * 4][64]
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
            for (int v = 0; v < 4; ++v) red[(w * RB * 4 + 4 * b + v) * 64 + lane] = facc[b][v];
        __syncthreads();
        if (w != 0) return;
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float s = red[(4 * b + v) * 64 + lane];
                for (int ww = 1; ww < nw; ++ww) s += red[(ww * RB * 4 + 4 * b + v) * 64 + lane];
                facc[b][v] = s;
            }
    }
    if (m >= M) return;
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        const int64_t nb = n0 + 16 * b + 4 * q;
        if (nb >= p.N) continue;
        float yv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) yv[v] = __builtin_fmaf(facc[b][v], sxm, bia[b][v]);
        // 4 consecutive bf16 of row m (8 bytes, aligned since N % 8 == 0)
        v2u o;
        o[0] = pack_bf16x2(yv[0], yv[1]);
        o[1] = pack_bf16x2(yv[2], yv[3]);
        *reinterpret_cast<v2u *>(p.y + (int64_t)m * p.N + nb) = o;
    }
}

struct Plan {
    int rb, nw;
    int64_t tiles;
};

// Rows per workgroup: 32 from N = 4096 on, else 16 (more workgroups for small N; each one
// re-reads the tokens, so not fewer rows than needed).  Wavefronts per workgroup: about
// TARGET_WAVES in all, but each with at least MIN_GROUPS groups.  Both measured on the decode
// shapes (N x K = 8192/1024/25600 x 5120, 5120 x 25600): fewer, longer-running wavefronts beat
// many short ones, whose prologue and final reduction dominate.
Plan plan(int64_t N, int K)
{
    Plan pl;
    pl.rb = N >= 4096 ? 2 : 1;
    pl.tiles = (N + 16 * pl.rb - 1) / (16 * pl.rb);
    int64_t nw = (TARGET_WAVES + pl.tiles - 1) / pl.tiles;
    const int G = (K + GS - 1) / GS;
    if (nw > G / MIN_GROUPS) nw = G / MIN_GROUPS;
    if (nw > MAX_NW) nw = MAX_NW;
    pl.nw = nw < 1 ? 1 : (int)nw;
    return pl;
}

template <int RB, bool G128>
hipError_t launch(const W4A8Params &p, const Plan &pl, hipStream_t stream)
{
    const size_t lds = (size_t)pl.nw * D * XSTAGE;
    hipLaunchKernelGGL((gemv_w4a8_kernel<RB, G128>), dim3((unsigned)pl.tiles), dim3(64 * pl.nw), lds, stream, p);
    return hipGetLastError();
}

} // namespace

size_t w4a8_packed_bytes(int64_t N, int K, int group)
{
    const int64_t tiles = (N + RT - 1) / RT;
    if (group == 128) return (size_t)(tiles * ((K + GS - 1) / GS) * BS128);
    return (size_t)(tiles * (K / GS) * BS);
}

hipError_t launch_pack_w4a8(const uint8_t *wq, const uint16_t *sw, int64_t N, int K, int group, uint8_t *out,
                            hipStream_t stream)
{
    if (group != 256 && group != 128) return hipErrorInvalidValue;
    if (K % group) return hipErrorInvalidValue;
    const bool g128 = group == 128;
    const int64_t nblocks = (N + RT - 1) / RT * ((K + GS - 1) / GS);
    const int64_t threads = nblocks * (CODE_BYTES / 16 + (g128 ? 2 : 1) * RT / 4);
    if (threads == 0) return hipSuccess;
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    if (g128)
        hipLaunchKernelGGL(pack_w4a8_kernel<true>, grid, block, 0, stream, wq, sw, out, N, K, nblocks);
    else
        hipLaunchKernelGGL(pack_w4a8_kernel<false>, grid, block, 0, stream, wq, sw, out, N, K, nblocks);
    return hipGetLastError();
}

int gemv_w4a8_waves(int64_t N, int K) { return plan(N, K).nw; }

hipError_t launch_gemv_w4a8(const int8_t *xq, const float *sx, const uint8_t *wp, const float *bias, void *y,
                            int64_t M, int64_t N, int K, int group, hipStream_t stream)
{
    if (M <= 0 || N <= 0) return hipSuccess;
    if ((group != 256 && group != 128) || K % group) return hipErrorInvalidValue;
    W4A8Params p;
    p.xq = xq;
    p.wp = wp;
    p.sx = sx;
    p.bias = bias;
    p.y = static_cast<uint16_t *>(y);
    p.N = N;
    p.M = (int)M;
    p.K = K;
    const Plan pl = plan(N, K);
    if (group == 128) return pl.rb == 2 ? launch<2, true>(p, pl, stream) : launch<1, true>(p, pl, stream);
    return pl.rb == 2 ? launch<2, false>(p, pl, stream) : launch<1, false>(p, pl, stream);
}

} // namespace convrot
