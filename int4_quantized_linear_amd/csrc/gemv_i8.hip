// gemv_i8.hip -- decode-shaped ConvRot linear (M <= 16 tokens), weight-bandwidth bound (gfx950).
//
// Same contraction and epilogue as the GEMM (acc = xq . wq^T, y = bf16(acc*sx*sw + bias)), for
// the few-token case: the conditioning pass of the text encoder on the pages runs at 12 tokens
// ("Qwen3-VL-32B-...-INT8-ConvRot部署优化", section 运行时验证指标, output (1, 12, 5120)), so every
// ConvRot linear there streams its whole INT8 weight once for 12 rows of work.
//
// Design: a workgroup (4 wavefronts) owns 64 weight rows and a slice of K, streamed in chunks
// of 256 bytes per row through NST LDS stages.  Loads go global -> LDS directly
// (buffer_load ... lds, 16 bytes per lane): one instruction moves 4 rows x 256 contiguous bytes,
// so HBM sees whole 128-byte lines and long runs per row.  The <= 16 token rows of the chunk
// (L2-resident) are staged the same way; tokens >= M and bytes past the slice read zeros through
// out-of-bounds buffer offsets.  In LDS, 16-byte chunk c of row r sits at position c ^ (r & 15),
// so the MFMA fragment reads (16 rows, same chunk) hit 16 distinct bank groups.  Wave w multiplies
// K-step w of every chunk for all 64 rows with v_mfma_i32_16x16x64_i8 (rows = weight rows,
// columns = tokens); the 4 waves' sums are added through LDS at the end.
//
// Split-K across workgroups (when the row tiles alone would not fill the chip): every split
// stores its int32 partial sums into its own workspace slot with device-coherent stores, waits
// for them to complete, then publishes a 64-bit arrival flag of its own (the call's generation
// tag and its complement) and, once that store has completed, reads the flags of all splits of
// its tile.  A split that sees every flag carrying the tag adds the other splits' partials to its
// own (exact integer sums), runs the epilogue and clears the flags.  Store-then-read on both
// sides guarantees that the last split to publish sees all flags; if several see them, they
// write identical results.  There is no shared counter, so splits never contend on one address,
// and stale workspace contents (other calls, other shapes, uninitialised memory) cannot match the
// tag: the workspace needs no zero-fill.  Clearing the flags keeps a replay of the same launch
// (same tag, e.g. from a captured graph) correct.  No cache-wide write-back/invalidate is needed:
// partials and flags bypass the non-coherent per-XCD caches.
#include <stdlib.h>

#include <atomic>
#include <chrono>

#include "device_common.hpp"
#include "launchers.hpp"

namespace convrot {
namespace {

constexpr int ROWS = 64;                 // weight rows per workgroup
constexpr int KC = 256;                  // K bytes per row per chunk (4 MFMA K-steps)
constexpr int NST = 4;                   // LDS stages (NST - 1 chunks in flight)
constexpr int WBYTES = ROWS * KC;        // 16 KiB of weights per stage
constexpr int XBYTES = 16 * KC;          // 4 KiB of tokens per stage
constexpr int STG = WBYTES + XBYTES;
constexpr int TARGET_WGS = 128;          // split-K only when fewer tiles than this (measured best)
constexpr int MAX_SPLITS = 64;           // one flag per lane of a wavefront
constexpr uint32_t OOB = 0x80000000u;    // buffer offset past num_records -> loads return 0
constexpr int NUM_RECORDS = 0x7ffffff0;

struct GemvParams {
    const int8_t *xq;
    const int8_t *wq;
    const float *sx;
    const float *sw;
    const float *bias;
    void *y;
    int32_t *part;                 // [splits, M, N] partial sums
    unsigned long long *flag;      // [tiles, splits] generation-tagged arrival flags
    int64_t N;
    int M, K, splits;
    unsigned gen;
};

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= n only.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }

template <Epi E>
__device__ __forceinline__ void gemv_store(const GemvParams &p, int m, int64_t n, int32_t acc, float coef, float bias)
{
    if constexpr (E == Epi::Int32) {
        static_cast<int32_t *>(p.y)[(int64_t)m * p.N + n] = acc;
    } else {
        const float v = __builtin_fmaf((float)acc, coef, bias);
        static_cast<uint16_t *>(p.y)[(int64_t)m * p.N + n] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
    }
}

template <Epi E>
__global__ void __launch_bounds__(256, 2) gemv_i8_kernel(GemvParams p)
{
    // NST * STG = 80 KiB, so two workgroups share a CU's 160 KiB of LDS; the split-K arrival
    // flag lives in the stage memory past the reduction area once the stages are done.
    __shared__ __attribute__((aligned(16))) uint8_t smem[NST * STG];
    int &last_flag = *reinterpret_cast<int *>(smem + 4 * 16 * 64 * 4);
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tile = blockIdx.x, split = blockIdx.y;
    const int64_t n0 = (int64_t)tile * ROWS;
    const int K = p.K;
    const int steps = K / 64;
    const int k_beg = (int)((int64_t)steps * split / p.splits) * 64;
    const int k_end = (int)((int64_t)steps * (split + 1) / p.splits) * 64;
    const int nchunks = (k_end - k_beg + KC - 1) / KC;

    // Load geometry.  Weights: instruction i (0..3) of wave w fills rows 16w+4i .. +3 of a stage,
    // lane -> row +lane/16 at 16-byte position lane%16, which holds chunk (lane%16) ^ (row & 15).
    // Tokens: wave w fills token rows 4w .. 4w+3 the same way.
    const int p16 = lane & 15, q4 = lane >> 4;
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(p.wq + n0 * K), (short)0, NUM_RECORDS, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(p.xq), (short)0, NUM_RECORDS, 0x00020000);
    uint32_t offw[4], kw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + 4 * i + q4;
        kw[i] = (uint32_t)(k_beg + 16 * (p16 ^ (r & 15)));
        offw[i] = n0 + r < p.N ? (uint32_t)(r * K) + kw[i] : OOB;
    }
    const int t = 4 * w + q4;
    const uint32_t kx = (uint32_t)(k_beg + 16 * (p16 ^ (t & 15)));
    const uint32_t offx = t < p.M ? (uint32_t)(t * K) + kx : OOB;

    auto issue = [&](int g) {
        uint8_t *st = smem + (g % NST) * STG;
        const uint32_t kk = (uint32_t)(g * KC);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t o = (offw[i] != OOB && kw[i] + kk < (uint32_t)k_end) ? offw[i] + kk : OOB;
            // weights are read once: nontemporal (aux bit 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void *)(st + (16 * w + 4 * i) * KC), 16, o, 0, 0, 2);
        }
        const uint32_t o = (offx != OOB && kx + kk < (uint32_t)k_end) ? offx + kk : OOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void *)(st + WBYTES + 4 * w * KC), 16, o, 0, 0, 0);
    };

    // Fragment addressing: wave w reads K-step w of a chunk; lane -> row/token lane%16, 16-byte
    // chunk 4w + lane/16 at position (4w + lane/16) ^ (lane%16).
    const int fpos = 16 * ((4 * w + q4) ^ p16);
    const int arow = p16 * KC + fpos;
    v4i acc[4] = {v4i{}, v4i{}, v4i{}, v4i{}};

    if (nchunks > 0) issue(0);
    if (nchunks > 1) issue(1);
    if (nchunks > 2) issue(2);

    // Outputs of this thread after the cross-wave reduction: entry idx = threadIdx + 256u of the
    // [16 values][64 lanes] accumulator image; the epilogue's scales and bias are fetched now,
    // behind the first chunks' loads, so that their latency hides under the main loop.
    int mm[4];
    int64_t nn[4];
    bool ok[4];
    float coef[4], bia[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int idx = threadIdx.x + 256 * u;
        const int v = idx >> 6, l = idx & 63;
        mm[u] = l & 15;
        nn[u] = n0 + 16 * (v >> 2) + 4 * (l >> 4) + (v & 3);
        ok[u] = mm[u] < p.M && nn[u] < p.N;
        coef[u] = 0.0f;
        bia[u] = 0.0f;
        if constexpr (E == Epi::Bf16) {
            // branch-free (clamped indices), so the loads are all in flight together
            const int mc = mm[u] < p.M ? mm[u] : p.M - 1;
            const int64_t nc = nn[u] < p.N ? nn[u] : p.N - 1;
            coef[u] = p.sx[mc] * p.sw[nc];
            bia[u] = p.bias ? p.bias[nc] : 0.0f;
        }
    }

    for (int g = 0; g < nchunks; ++g) {
        // chunk g has landed once at most the loads of chunks g+1, g+2 (5 per wave each) remain
        if (g + 2 < nchunks) __builtin_amdgcn_s_waitcnt(waitcnt_vm(10));
        else if (g + 1 < nchunks) __builtin_amdgcn_s_waitcnt(waitcnt_vm(5));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        // Barrier without a memory fence: a fence would make the compiler wait for every load in
        // flight (vmcnt 0) and serialise the pipeline.  The explicit vmcnt wait above covers this
        // wave's chunk-g loads, lgkmcnt(0) retires its LDS reads of the stage about to be refilled.
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (g + 3 < nchunks) issue(g + 3);
        const uint8_t *st = smem + (g % NST) * STG;
        const v4i xb = *reinterpret_cast<const v4i *>(st + WBYTES + arow);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const v4i wa = *reinterpret_cast<const v4i *>(st + 16 * b * KC + arow);
            acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wa, xb, acc[b], 0, 0, 0);
        }
    }

    // 16x16 accumulator layout: lane holds token m = lane%16 and weight rows 4*(lane/16) + v.
    __syncthreads();                         // all waves are done with the stages
    int32_t *red = reinterpret_cast<int32_t *>(smem);   // [4 waves][16 values][64 lanes]
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[(w * 16 + 4 * b + v) * 64 + lane] = acc[b][v];
    __syncthreads();

    int32_t sum[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int idx = threadIdx.x + 256 * u;
        sum[u] = red[idx] + red[1024 + idx] + red[2048 + idx] + red[3072 + idx];
    }

    if (p.splits == 1) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (ok[u]) gemv_store<E>(p, mm[u], nn[u], sum[u], coef[u], bia[u]);
        return;
    }

    const int64_t MN = (int64_t)p.M * p.N;
#pragma unroll
    for (int u = 0; u < 4; ++u)
        if (ok[u])
            __hip_atomic_store(&p.part[split * MN + (int64_t)mm[u] * p.N + nn[u]], sum[u], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);     // this thread's partial stores have completed
    __syncthreads();
    if (w == 0) {
        const unsigned long long tag = ((unsigned long long)p.gen << 32) | (unsigned)~p.gen;
        unsigned long long *fl = p.flag + (int64_t)tile * p.splits;
        if (lane == 0) __hip_atomic_store(fl + split, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0); // the flag store has completed before any flag is read
        const bool seen = lane >= p.splits || lane == split ||
                          __hip_atomic_load(fl + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag;
        const bool all = __builtin_amdgcn_ballot_w64(!seen) == 0;
        // every split has arrived: clear the flags (all were written already) for a replay
        if (all && lane < p.splits) __hip_atomic_store(fl + lane, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (lane == 0) last_flag = all;
    }
    __syncthreads();
    if (!last_flag) return;
    // Sum the other splits' partials (integer addition: exact in any order).  The loads of a
    // batch of 8 splits x 4 outputs are independent, so they are in flight together instead of
    // paying one memory round trip per split.
    const int32_t *part[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) part[u] = p.part + (ok[u] ? (int64_t)mm[u] * p.N + nn[u] : 0);
    for (int s0 = 0; s0 < p.splits; s0 += 8) {
        int32_t v[4][8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int s = s0 + j;
            const bool use = s < p.splits && s != split;
#pragma unroll
            for (int u = 0; u < 4; ++u)
                v[u][j] = (use && ok[u]) ? __hip_atomic_load(part[u] + s * MN, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                         : 0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < 8; ++j) sum[u] += v[u][j];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
        if (ok[u]) gemv_store<E>(p, mm[u], nn[u], sum[u], coef[u], bia[u]);
}

int forced_splits()
{
    static const int v = [] {
        const char *e = getenv("CONVROT_GEMV_SPLITS");
        return e ? atoi(e) : 0;
    }();
    return v;
}

unsigned next_generation()
{
    // Seeded per process so that leftovers from another process never carry the current tag.
    static std::atomic<unsigned> gen{(unsigned)std::chrono::steady_clock::now().time_since_epoch().count() | 1u};
    unsigned g = gen.fetch_add(1) + 1;
    return g ? g : gen.fetch_add(1) + 1;
}

} // namespace

int gemv_i8_splits(int64_t N, int K)
{
    const int64_t tiles = (N + ROWS - 1) / ROWS;
    int s = forced_splits() > 0 ? forced_splits() : (int)((TARGET_WGS + tiles - 1) / tiles);
    int smax = K / KC > 1 ? K / KC : 1;            // at least one full chunk per split
    if (smax > MAX_SPLITS) smax = MAX_SPLITS;
    if (s > smax) s = smax;
    return s < 1 ? 1 : s;
}

size_t gemv_i8_workspace_bytes(int64_t M, int64_t N, int K)
{
    const int64_t tiles = (N + ROWS - 1) / ROWS;
    const int s = gemv_i8_splits(N, K);
    if (s == 1) return 0;
    return (size_t)(tiles * s * 8 + (int64_t)s * M * N * 4);
}

hipError_t launch_gemv_i8(const int8_t *xq, const int8_t *wq, const float *sx, const float *sw, const float *bias,
                          void *y, Epi epi, int64_t M, int64_t N, int K, void *ws, hipStream_t stream)
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
    p.splits = gemv_i8_splits(N, K);
    const int64_t tiles = (N + ROWS - 1) / ROWS;
    p.flag = static_cast<unsigned long long *>(ws);
    p.part = reinterpret_cast<int32_t *>(static_cast<uint8_t *>(ws) + tiles * p.splits * 8);
    p.gen = next_generation();
    const dim3 grid((unsigned)tiles, (unsigned)p.splits), block(256);
    if (epi == Epi::Int32)
        hipLaunchKernelGGL(gemv_i8_kernel<Epi::Int32>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(gemv_i8_kernel<Epi::Bf16>, grid, block, 0, stream, p);
    return hipGetLastError();
}

} // namespace convrot
