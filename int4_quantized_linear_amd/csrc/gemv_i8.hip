// gemv_i8.hip -- decode-shaped ConvRot linear (M <= 16 tokens), weight-bandwidth bound (gfx950).
//
// Same contraction and epilogue as the GEMM (acc = xq . wq^T, y = bf16(acc*sx*sw + bias)), for
// the few-token case: the conditioning pass of the text encoder on the pages runs at 12 tokens
// ("Qwen3-VL-32B-...-INT8-ConvRot部署优化", section 运行时验证指标, output (1, 12, 5120)), so every
// ConvRot linear there streams its whole INT8 weight once for 12 rows of work.
//
// Design: a workgroup (4 wavefronts) owns 64 weight rows and a slice of K.  A wavefront streams
// its rows as 4 blocks of v_mfma_i32_16x16x64_i8 (MFMA rows = weight rows, columns = tokens;
// token columns >= M read zeros), so the matrix core does the multiply-adds and the VALU stays
// free.  Each iteration issues UNROLL K steps (5 x 16-byte loads per lane per step) before the
// first MFMA; the 4 wavefronts interleave K steps and are summed through LDS.
//
// Split-K across workgroups (only when there are too few row tiles to fill the chip): every
// split stores its int32 partial sums into its own workspace slot with device-coherent stores,
// waits for them to complete, and bumps a per-tile arrival counter.  The counter carries the
// call's 32-bit generation tag in its upper half, so a stale value from any earlier call (or
// uninitialised memory) simply restarts the count: the workspace needs no zero-fill.  The last
// split to arrive adds the partials in split order (exact, deterministic) and runs the epilogue.
// No cache-wide write-back/invalidate is needed: partials and counter bypass the non-coherent
// per-XCD caches.
#include <stdlib.h>

#include <atomic>
#include <chrono>

#include "device_common.hpp"
#include "launchers.hpp"

namespace convrot {
namespace {

constexpr int ROWS = 64;     // weight rows per workgroup
constexpr int STEP = 64;     // K bytes per MFMA step
constexpr int UNROLL = 4;    // K steps per wavefront per iteration

struct GemvParams {
    const int8_t *xq;
    const int8_t *wq;
    const float *sx;
    const float *sw;
    const float *bias;
    void *y;
    int32_t *part;                 // [splits, M, N] partial sums
    unsigned long long *cnt;       // [tiles] generation-tagged arrival counters
    int64_t N;
    int M, K, splits;
    unsigned gen;
};

template <Epi E>
__device__ __forceinline__ void gemv_store(const GemvParams &p, int m, int64_t n, int32_t acc)
{
    if constexpr (E == Epi::Int32) {
        static_cast<int32_t *>(p.y)[(int64_t)m * p.N + n] = acc;
    } else {
        const float b = p.bias ? p.bias[n] : 0.0f;
        const float v = __builtin_fmaf((float)acc, p.sx[m] * p.sw[n], b);
        static_cast<uint16_t *>(p.y)[(int64_t)m * p.N + n] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
    }
}

template <Epi E>
__global__ void __launch_bounds__(256) gemv_i8_kernel(GemvParams p)
{
    __shared__ int32_t red[4][16 * 64];
    __shared__ int last_flag;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int tile = blockIdx.x, split = blockIdx.y;
    const int64_t n0 = (int64_t)tile * ROWS;
    const int steps = p.K / STEP;
    const int s_beg = (int)((int64_t)steps * split / p.splits);
    const int s_end = (int)((int64_t)steps * (split + 1) / p.splits);

    const int r16 = lane & 15, q = lane >> 4;
    const int8_t *wrow[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        int64_t n = n0 + 16 * b + r16;
        n = n < p.N ? n : p.N - 1;      // rows >= N are computed but never stored
        wrow[b] = p.wq + n * p.K + 16 * q;
    }
    const bool xok = r16 < p.M;
    const int8_t *xrow = p.xq + (int64_t)(xok ? r16 : 0) * p.K + 16 * q;

    v4i acc[4] = {v4i{}, v4i{}, v4i{}, v4i{}};
    for (int s = s_beg + w; s < s_end; s += 4 * UNROLL) {
        v4i fw[UNROLL][4], fx[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const bool ok = s + 4 * u < s_end;
            const int k = (s + 4 * u) * STEP;
#pragma unroll
            for (int b = 0; b < 4; ++b)
                fw[u][b] = ok ? __builtin_nontemporal_load(reinterpret_cast<const v4i *>(wrow[b] + k)) : v4i{};
            fx[u] = (ok && xok) ? *reinterpret_cast<const v4i *>(xrow + k) : v4i{};
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fw[u][b], fx[u], acc[b], 0, 0, 0);
    }

    // 16x16 accumulator layout: lane holds token m = lane%16 and weight rows 4*(lane/16) + v.
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v) red[w][(4 * b + v) * 64 + lane] = acc[b][v];
    __syncthreads();

    int32_t sum[4];
    int mm[4];
    int64_t nn[4];
    bool ok[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int idx = threadIdx.x + 256 * u;
        sum[u] = red[0][idx] + red[1][idx] + red[2][idx] + red[3][idx];
        const int v = idx >> 6, l = idx & 63;
        mm[u] = l & 15;
        nn[u] = n0 + 16 * (v >> 2) + 4 * (l >> 4) + (v & 3);
        ok[u] = mm[u] < p.M && nn[u] < p.N;
    }

    if (p.splits == 1) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (ok[u]) gemv_store<E>(p, mm[u], nn[u], sum[u]);
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
    if (threadIdx.x == 0) {
        unsigned long long old = __hip_atomic_load(&p.cnt[tile], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        unsigned long long nw;
        do {
            nw = ((unsigned)(old >> 32) == p.gen) ? old + 1 : (((unsigned long long)p.gen << 32) | 1ull);
        } while (!__hip_atomic_compare_exchange_strong(&p.cnt[tile], &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT));
        last_flag = (int)(nw & 0xffffffffull) == p.splits;
        // Every split of this call has arrived: clear the counter so that a replay of the same
        // launch (same generation tag, e.g. from a captured graph) starts counting from zero.
        if (last_flag) __hip_atomic_store(&p.cnt[tile], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last_flag) return;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (!ok[u]) continue;
        const int64_t o = (int64_t)mm[u] * p.N + nn[u];
        int32_t total = 0;
        for (int s = 0; s < p.splits; ++s)
            total += __hip_atomic_load(&p.part[s * MN + o], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        gemv_store<E>(p, mm[u], nn[u], total);
    }
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
    const int steps = K / STEP;
    int s = forced_splits() > 0 ? forced_splits() : (int)((1024 + tiles - 1) / tiles);
    const int smax = steps / (4 * UNROLL) > 1 ? steps / (4 * UNROLL) : 1;
    if (s > smax) s = smax;
    if (s > steps) s = steps;
    return s < 1 ? 1 : s;
}

size_t gemv_i8_workspace_bytes(int64_t M, int64_t N, int K)
{
    const int64_t tiles = (N + ROWS - 1) / ROWS;
    const int s = gemv_i8_splits(N, K);
    if (s == 1) return 0;
    return (size_t)(tiles * 8 + (int64_t)s * M * N * 4);
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
    p.cnt = static_cast<unsigned long long *>(ws);
    p.part = reinterpret_cast<int32_t *>(static_cast<uint8_t *>(ws) + tiles * 8);
    p.gen = next_generation();
    const dim3 grid((unsigned)tiles, (unsigned)p.splits), block(256);
    if (epi == Epi::Int32)
        hipLaunchKernelGGL(gemv_i8_kernel<Epi::Int32>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(gemv_i8_kernel<Epi::Bf16>, grid, block, 0, stream, p);
    return hipGetLastError();
}

} // namespace convrot
