// gemv_w4a8.hip -- decode-shaped W4A8 ConvRot linear (M <= 16 tokens), weight-bandwidth bound.
//
// INT4 weights (one fp16 scale per (row, 256-channel group), two codes per byte) against INT8
// tokens (one fp32 scale per token), both rotated by the same grouped Hadamard (the W4A8
// ConvRot variant: 4-bit weights, 8-bit activations, "MiniMax-H3-W4A8-ConvRot" pages):
//   y[m,n] = bf16( sx[m] * sum_j sw[j,n] * (sum_{k in group j} qx[m,k] * cw[n,k]) + bias[n] )
// Half the weight bytes of the INT8 GEMV for the same shape.
//
// Design: a workgroup (4 wavefronts) owns 64 weight rows and a slice of the K groups, streamed
// one group (256 codes = 128 packed bytes per row) per chunk through NST LDS stages with
// buffer_load ... lds (one instruction moves 8 rows x 128 bytes).  Wavefront w owns rows
// 16w .. 16w+15 and all four 64-code K-steps of a chunk, so a group's integer dot products
// finish inside one wavefront and are scaled right away (no cross-wave reduction):
//  * A operand (weights): 8 packed bytes per lane (ds_read_b64) widened to 16 int8 codes x16 in
//    natural order (low nibble = even channel), 5 VALU per packed dword;
//  * B operand (tokens): 16 int8 codes per lane (ds_read_b128); tokens >= M read zeros;
//  * v_mfma_i32_16x16x64_i8 per K-step (rows = weight rows, columns = tokens); after the group:
//    facc += float(iacc) * sw / 16, and the next group's first MFMA starts from zero.
// LDS swizzles: weight row r keeps 16-byte chunk c at c ^ ((r >> 1) & 7), token row t keeps
// chunk c at c ^ (t & 15); both make the fragment reads conflict-free.  The group's 16 scales of
// a wavefront arrive with the chunk by a 2-byte load-to-LDS (one scale per dword).
// Split-K across workgroups when there are too few row tiles: fp32 partials, per-split
// generation-tagged arrival flags, the split that sees all flags adds the partials in split
// order (same protocol as the INT8 GEMV).
#include <stdlib.h>

#include <atomic>
#include <chrono>

#include "device_common.hpp"
#include "launchers.hpp"

namespace convrot {
namespace {

constexpr int ROWS = 64;
constexpr int GC = 256;                  // codes per chunk (= one scale group)
constexpr int KB = GC / 2;               // packed bytes per row per chunk
constexpr int NST = 4;
constexpr int WBYTES = ROWS * KB;        // 8 KiB
constexpr int XBYTES = 16 * GC;          // 4 KiB
constexpr int SBYTES = 4 * 256;          // one 256-byte scale block per wavefront
constexpr int STG = WBYTES + XBYTES + SBYTES;
constexpr int TARGET_WGS = 256;
constexpr int MAX_SPLITS = 64;
constexpr uint32_t OOB = 0x80000000u;
constexpr int NUM_RECORDS = 0x7ffffff0;

struct W4A8Params {
    const int8_t *xq;
    const uint8_t *wq;       // packed [N, K/2]
    const float *sx;
    const uint16_t *sw;      // [G, N] fp16
    const float *bias;
    uint16_t *y;
    float *part;             // [splits, M, N]
    unsigned long long *flag;
    int64_t N;
    int M, K, splits;
    unsigned gen;
};

typedef __attribute__((address_space(3))) void lds_void;

constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }

// 8 packed bytes (16 codes, even channel in the low nibble) -> 16 bytes 16*c in channel order.
__device__ __forceinline__ v4i widen16(uint2 d)
{
    v4i o;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t p = h ? d.y : d.x;
        const uint32_t lo = (p << 4) & 0xF0F0F0F0u;    // c0 c2 c4 c6 (x16)
        const uint32_t hi = p & 0xF0F0F0F0u;           // c1 c3 c5 c7 (x16)
        o[2 * h] = (int)__builtin_amdgcn_perm(hi, lo, 0x05010400u);       // c0 c1 c2 c3
        o[2 * h + 1] = (int)__builtin_amdgcn_perm(hi, lo, 0x07030602u);   // c4 c5 c6 c7
    }
    return o;
}

__global__ void __launch_bounds__(256, 3) gemv_w4a8_kernel(W4A8Params p)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[NST * STG];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tile = blockIdx.x, split = blockIdx.y;
    const int64_t n0 = (int64_t)tile * ROWS;
    const int K = p.K;
    const int G = K / GC;
    const int g_beg = (int)((int64_t)G * split / p.splits);
    const int g_end = (int)((int64_t)G * (split + 1) / p.splits);
    const int nchunks = g_end - g_beg;

    // Weights: instruction i (0..1) of wave w fills rows 8*(2w+i) .. +7, lane -> row +lane/8,
    // 16-byte position lane%8 holding chunk (lane%8) ^ ((row >> 1) & 7).
    const int Kh = K / 2;
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p.wq + n0 * Kh), (short)0, NUM_RECORDS, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(p.xq), (short)0, NUM_RECORDS, 0x00020000);
    uint32_t offw[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 8 * (2 * w + i) + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        offw[i] = n0 + r < p.N ? (uint32_t)(r * Kh + g_beg * KB + 16 * c) : OOB;
    }
    // Tokens: wave w fills token rows 4w .. 4w+3, lane -> token +lane/16, position lane%16
    // holding chunk (lane%16) ^ token.
    const int t = 4 * w + (lane >> 4);
    const uint32_t offx = t < p.M ? (uint32_t)(t * K + g_beg * GC + 16 * ((lane & 15) ^ (t & 15))) : OOB;
    // Scales of this wave's 16 rows for group j: sw[j*N + n0 + 16w + lane], lanes >= 16 off.
    const int64_t srow = n0 + 16 * w + lane;
    const bool sok = lane < 16 && srow < p.N;

    auto issue = [&](int c) {
        uint8_t *st = smem + (c % NST) * STG;
        const uint32_t kw = (uint32_t)(c * KB), kx = (uint32_t)(c * GC);
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(st + (2 * w + i) * 1024), 16,
                                                     offw[i] == OOB ? OOB : offw[i] + kw, 0, 0, 2);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(st + WBYTES + w * 1024), 16,
                                                 offx == OOB ? OOB : offx + kx, 0, 0, 0);
        // one fp16 scale per lane, zero-extended into a dword of this wave's scale block
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t *>(p.sw + (int64_t)(g_beg + c) * p.N), (short)0, (int)(2 * p.N), 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(st + WBYTES + XBYTES + w * 256), 2,
                                                 sok ? (uint32_t)(2 * srow) : OOB, 0, 0, 0);
    };

    // Fragments: A row 16w + lane%16, packed bytes 32kk + 8*(lane/16) = 16-byte chunk
    // 2kk + (lane/16)/2, half (lane/16)&1; B token lane%16, chunk 4kk + lane/16.
    const int fr = lane & 15, fq = lane >> 4;
    const int arow = 16 * w + fr;
    const int abase = arow * KB + 8 * (fq & 1);
    const int aswz = (arow >> 1) & 7;
    const int bbase = WBYTES + fr * GC;
    float facc[4] = {0.f, 0.f, 0.f, 0.f};

    if (nchunks > 0) issue(0);
    if (nchunks > 1) issue(1);
    if (nchunks > 2) issue(2);
    for (int c = 0; c < nchunks; ++c) {
        if (c + 2 < nchunks) __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));
        else if (c + 1 < nchunks) __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        // raw barrier: __syncthreads()'s fence would wait for every load in flight
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (c + 3 < nchunks) issue(c + 3);
        const uint8_t *st = smem + (c % NST) * STG;
        v4i iacc = v4i{};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int ca = 2 * kk + (fq >> 1);
            // an ext-vector load keeps its type-based alias info, so the compiler adds no vmcnt(0)
            // for the loads-to-LDS in flight (the explicit waits above order them)
            const v2u pv = *reinterpret_cast<const v2u *>(st + abase + 16 * (ca ^ aswz));
            const uint2 pa = make_uint2(pv[0], pv[1]);
            const v4i xb = *reinterpret_cast<const v4i *>(st + bbase + 16 * ((4 * kk + fq) ^ fr));
            iacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(widen16(pa), xb, iacc, 0, 0, 0);
        }
        // 16x16 layout: lane holds token lane%16 and rows 4*(lane/16) + v of the wave's 16
        const v4u s4 = *reinterpret_cast<const v4u *>(st + WBYTES + XBYTES + w * 256 + 16 * fq);
#pragma unroll
        for (int v = 0; v < 4; ++v)
            facc[v] = __builtin_fmaf((float)iacc[v], (float)__ushort_as_half((unsigned short)s4[v]) * 0.0625f, facc[v]);
    }

    const int m = fr;
    const bool mok = m < p.M;
    int64_t nn[4];
    bool ok[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        nn[v] = n0 + 16 * w + 4 * fq + v;
        ok[v] = mok && nn[v] < p.N;
    }
    auto store = [&](int v, float acc) {
        const float b = p.bias ? p.bias[nn[v]] : 0.0f;
        const float yv = __builtin_fmaf(acc, p.sx[m], b);
        p.y[(int64_t)m * p.N + nn[v]] = (uint16_t)(pack_bf16x2(yv, 0.0f) & 0xffffu);
    };
    if (p.splits == 1) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
            if (ok[v]) store(v, facc[v]);
        return;
    }

    // split-K: publish fp32 partials, then the arrival flag; whoever sees every flag finishes
    // in the (now idle) stage memory: a second LDS object would give the stage reads alias scopes
    // under which the compiler waits for every load-to-LDS in flight before each read
    int &last_flag = *reinterpret_cast<int *>(smem);
    const int64_t MN = (int64_t)p.M * p.N;
#pragma unroll
    for (int v = 0; v < 4; ++v)
        if (ok[v])
            __hip_atomic_store(&p.part[split * MN + (int64_t)m * p.N + nn[v]], facc[v], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (w == 0) {
        const unsigned long long tag = ((unsigned long long)p.gen << 32) | (unsigned)~p.gen;
        unsigned long long *fl = p.flag + (int64_t)tile * p.splits;
        if (lane == 0) __hip_atomic_store(fl + split, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        const bool seen = lane >= p.splits || lane == split ||
                          __hip_atomic_load(fl + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag;
        const bool all = __builtin_amdgcn_ballot_w64(!seen) == 0;
        if (all && lane < p.splits) __hip_atomic_store(fl + lane, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) last_flag = all;
    }
    __syncthreads();
    if (!last_flag) return;
    // fp32 partials summed in split order (deterministic)
    for (int v = 0; v < 4; ++v) {
        if (!ok[v]) continue;
        const float *pp = p.part + (int64_t)m * p.N + nn[v];
        float tot = 0.0f;
        for (int s0 = 0; s0 < p.splits; s0 += 8) {
            float vals[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                vals[j] = (s0 + j < p.splits) ? __hip_atomic_load(pp + (s0 + j) * MN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                              : 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) tot += vals[j];
        }
        store(v, tot);
    }
}

unsigned next_generation()
{
    static std::atomic<unsigned> gen{(unsigned)std::chrono::steady_clock::now().time_since_epoch().count() | 1u};
    unsigned g = gen.fetch_add(1) + 1;
    return g ? g : gen.fetch_add(1) + 1;
}

} // namespace

int gemv_w4a8_splits(int64_t N, int K)
{
    const int64_t tiles = (N + ROWS - 1) / ROWS;
    int s = (int)((TARGET_WGS + tiles - 1) / tiles);
    int smax = K / GC;
    if (smax > MAX_SPLITS) smax = MAX_SPLITS;
    if (s > smax) s = smax;
    return s < 1 ? 1 : s;
}

size_t gemv_w4a8_workspace_bytes(int64_t M, int64_t N, int K)
{
    const int64_t tiles = (N + ROWS - 1) / ROWS;
    const int s = gemv_w4a8_splits(N, K);
    if (s == 1) return 0;
    return (size_t)(tiles * s * 8 + (int64_t)s * M * N * 4);
}

hipError_t launch_gemv_w4a8(const int8_t *xq, const float *sx, const uint8_t *wq, const uint16_t *sw, const float *bias,
                            void *y, int64_t M, int64_t N, int K, void *ws, hipStream_t stream)
{
    if (M <= 0 || N <= 0) return hipSuccess;
    W4A8Params p;
    p.xq = xq;
    p.wq = wq;
    p.sx = sx;
    p.sw = sw;
    p.bias = bias;
    p.y = static_cast<uint16_t *>(y);
    p.N = N;
    p.M = (int)M;
    p.K = K;
    p.splits = gemv_w4a8_splits(N, K);
    const int64_t tiles = (N + ROWS - 1) / ROWS;
    p.flag = static_cast<unsigned long long *>(ws);
    p.part = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + tiles * p.splits * 8);
    p.gen = next_generation();
    hipLaunchKernelGGL(gemv_w4a8_kernel, dim3((unsigned)tiles, (unsigned)p.splits), dim3(256), 0, stream, p);
    return hipGetLastError();
}

} // namespace convrot
