// gemv_i8.hip -- decode-shaped ConvRot linear (M <= 16 tokens), weight-bandwidth bound (gfx950).
//
// Same contraction and epilogue as the GEMM (acc = xq . wq^T, y = bf16(acc*sx*sw + bias)), for
// the few-token case: the conditioning pass of the text encoder on the pages runs at 12 tokens
// ("Qwen3-VL-32B-...-INT8-ConvRot部署优化", section 运行时验证指标, output (1, 12, 5120)), so every
// ConvRot linear there streams its whole INT8 weight once for 12 rows of work.
//
// Design: each workgroup (4 wavefronts) owns 64 weight rows and a slice of K.  A wavefront
// streams its 64 rows as 4 blocks of v_mfma_i32_16x16x64_i8 (MFMA rows = weight rows, columns =
// tokens; token columns >= M read zeros), so the tensor core does the multiply-adds and the
// VALU stays free; each lane keeps 5 x 16-byte loads per 64-byte K step and several steps in
// flight.  The 4 wavefronts interleave K steps and are summed through LDS.  When K is split
// over several workgroups, partial sums are added exactly (int32 atomics, so the result does not
// depend on arrival order) into a workspace that was zero-filled just before the launch, and the
// last workgroup to arrive on a row tile (arrival counter) applies the epilogue.
#include "device_common.hpp"
#include "launchers.hpp"

namespace convrot {
namespace {

constexpr int ROWS = 64;     // weight rows per workgroup
constexpr int STEP = 64;     // K bytes per MFMA step
constexpr int UNROLL = 4;    // K steps in flight per wavefront

struct GemvParams {
    const int8_t *xq;
    const int8_t *wq;
    const float *sx;
    const float *sw;
    const float *bias;
    void *y;
    int32_t *ws_acc;       // [M, N] partial sums, zero on entry
    uint32_t *ws_cnt;      // [tiles] arrival counters, zero on entry
    int64_t N;
    int M, K, splits;
};

template <Epi E>
__device__ __forceinline__ void gemv_store(const GemvParams &p, int m, int64_t n, int32_t acc)
{
    if constexpr (E == Epi::Int32) {
        static_cast<int32_t *>(p.y)[(int64_t)m * p.N + n] = acc;
    } else {
        const float b = p.bias ? p.bias[n] : 0.0f;
        const float v = __builtin_fmaf((float)acc, p.sx[m] * p.sw[n], b);
        const uint32_t pk = pack_bf16x2(v, 0.0f);
        static_cast<uint16_t *>(p.y)[(int64_t)m * p.N + n] = (uint16_t)(pk & 0xffffu);
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
    // weight rows of the 4 blocks (clamped in range; rows >= N are never stored)
    const int8_t *wrow[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        int64_t n = n0 + 16 * b + r16;
        n = n < p.N ? n : p.N - 1;
        wrow[b] = p.wq + n * p.K + 16 * q;
    }
    const bool xok = r16 < p.M;
    const int8_t *xrow = p.xq + (int64_t)(xok ? r16 : 0) * p.K + 16 * q;

    v4i acc[4] = {v4i{}, v4i{}, v4i{}, v4i{}};
    int s = s_beg + w;
    for (; s + 4 * (UNROLL - 1) < s_end; s += 4 * UNROLL) {
        v4i fw[UNROLL][4], fx[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int k = (s + 4 * u) * STEP;
#pragma unroll
            for (int b = 0; b < 4; ++b) fw[u][b] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(wrow[b] + k));
            fx[u] = xok ? *reinterpret_cast<const v4i *>(xrow + k) : v4i{};
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fw[u][b], fx[u], acc[b], 0, 0, 0);
    }
    for (; s < s_end; s += 4) {
        const int k = s * STEP;
        v4i fw[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) fw[b] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(wrow[b] + k));
        const v4i fx = xok ? *reinterpret_cast<const v4i *>(xrow + k) : v4i{};
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fw[b], fx, acc[b], 0, 0, 0);
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

#pragma unroll
    for (int u = 0; u < 4; ++u)
        if (ok[u]) atomicAdd(&p.ws_acc[(int64_t)mm[u] * p.N + nn[u]], sum[u]);
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) last_flag = atomicAdd(&p.ws_cnt[tile], 1u) == (uint32_t)(p.splits - 1);
    __syncthreads();
    if (!last_flag) return;
    __threadfence();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (!ok[u]) continue;
        int32_t *slot = &p.ws_acc[(int64_t)mm[u] * p.N + nn[u]];
        gemv_store<E>(p, mm[u], nn[u], __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    }
}

int gemv_splits(int64_t N, int K)
{
    const int tiles = (int)((N + ROWS - 1) / ROWS);
    const int steps = K / STEP;
    static int forced = -1;
    if (forced < 0) {
        const char *e = getenv("CONVROT_GEMV_SPLITS");
        forced = e ? atoi(e) : 0;
    }
    int s = forced > 0 ? forced : (1024 + tiles - 1) / tiles;
    const int smax = steps / 8 > 1 ? steps / 8 : 1;
    if (s > smax) s = smax;
    if (s < 1) s = 1;
    return s;
}

} // namespace

size_t gemv_i8_workspace_bytes(int64_t M, int64_t N)
{
    const int64_t tiles = (N + ROWS - 1) / ROWS;
    return (size_t)(M * N * 4 + tiles * 4);
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
    p.splits = gemv_splits(N, K);
    p.ws_acc = static_cast<int32_t *>(ws);
    p.ws_cnt = reinterpret_cast<uint32_t *>(static_cast<int32_t *>(ws) + M * N);
    const dim3 grid((unsigned)((N + ROWS - 1) / ROWS), (unsigned)p.splits), block(256);
    if (epi == Epi::Int32)
        hipLaunchKernelGGL(gemv_i8_kernel<Epi::Int32>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(gemv_i8_kernel<Epi::Bf16>, grid, block, 0, stream, p);
    return hipGetLastError();
}

} // namespace convrot
