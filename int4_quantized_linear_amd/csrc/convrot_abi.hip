// convrot_abi.hip -- host side of the libconvrot C-ABI: argument validation, dispatch by
// shape, workspace layout and error reporting.  Every precondition is checked before the first
// HIP call, so a rejected call enqueues nothing.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "../../include/convrot.h"
#include "launchers.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = std::string(convrot_status_string(code)) + ": " + buf;
    return code;
}

bool pow2_group(int g) { return g >= 1 && g <= 256 && (g & (g - 1)) == 0; }
int log2i(int g)
{
    int l = 0;
    while ((1 << l) < g) ++l;
    return l;
}
bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

int check_shape(int64_t M, int64_t N, int64_t K, int group, const char *who)
{
    if (M < 0 || N < 0 || M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31))
        return fail(CONVROT_ERR_SHAPE, "%s: M=%lld N=%lld must be in [0, 2^31)", who, (long long)M, (long long)N);
    if (K < 64 || K > CONVROT_MAX_K || K % 64)
        return fail(CONVROT_ERR_SHAPE, "%s: K=%lld must be a multiple of 64 in [64, %d]", who, (long long)K,
                    CONVROT_MAX_K);
    if (!pow2_group(group))
        return fail(CONVROT_ERR_GROUP, "%s: group=%d must be a power of two in [1, 256]", who, group);
    if (K % group) return fail(CONVROT_ERR_SHAPE, "%s: K=%lld is not a multiple of group=%d", who, (long long)K, group);
    return CONVROT_OK;
}

// N limit of the tiled GEMMs (their 32-row output blocks use 32-bit byte offsets).
int check_gemm_n(int64_t N, const char *who)
{
    if (N >= CONVROT_GEMM_MAX_N)
        return fail(CONVROT_ERR_SHAPE, "%s: N=%lld; the tiled GEMM (M > 16, or W4A4) needs N < %d", who, (long long)N,
                    CONVROT_GEMM_MAX_N);
    return CONVROT_OK;
}

// One cached answer per device: is it gfx950?
int check_device()
{
    static std::mutex mu;
    static int known[64];   // 0 unknown, 1 ok, 2 wrong arch
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(CONVROT_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(CONVROT_ERR_DEVICE, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lk(mu);
    if (!known[dev]) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return fail(CONVROT_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        known[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (known[dev] == 2) return fail(CONVROT_ERR_DEVICE, "device %d is %s, libconvrot is built for gfx950", dev, prop.gcnArchName);
    }
    return known[dev] == 1 ? CONVROT_OK : fail(CONVROT_ERR_DEVICE, "device %d is not gfx950", dev);
}

int hip_status(hipError_t e, const char *what)
{
    return e == hipSuccess ? CONVROT_OK : fail(CONVROT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Workspace layout, each region 256-byte aligned; all of it is scratch (no initial contents):
//   bits 8: [xq int8 M*K][x_scale fp32 M]
//   bits 4: [xq packed M*K/2][x_scale fp16 (K/128)*M, enough for either INT4 group][FP6 tiles of
//           both operands]
struct WsLayout {
    size_t xq = 0, xs = 0, tiles = 0, part = 0, total = 0;
};

WsLayout ws_layout(int64_t M, int64_t N, int64_t K, int bits)
{
    WsLayout L;
    size_t off = 0;
    if (bits == 8) {
        L.xq = off;
        off += round256((size_t)(M * K));
        L.xs = off;
        off += round256((size_t)M * 4);
        // optional: the split-K tail's int32 partial sums (GEMM path only)
        L.part = off;
        if (M > 16) off += round256(convrot::gemm_i8_split_bytes(M, N, (int)K));
    } else {
        L.xq = off;
        off += round256((size_t)(M * K / 2));
        L.xs = off;
        off += round256((size_t)(M * ((K + 127) / 128) * 2));
        L.tiles = off;
        off += round256(convrot::w4a4_tiled_bytes(M, N, (int)K));
    }
    L.total = off;
    return L;
}

// W4A8 workspace: [xq int8 M*K][x_scale fp32 M], used when the entry point quantizes x itself.
WsLayout ws_layout_w4a8(int64_t M, int64_t K)
{
    WsLayout L;
    size_t off = 0;
    L.xq = off;
    off += round256((size_t)(M * K));
    L.xs = off;
    off += round256((size_t)M * 4);
    L.total = off;
    return L;
}

int quantize_common(const void *x, int dtype, int64_t R, int64_t K, int group, int bits, void *q, void *scale,
                    hipStream_t stream, const char *who)
{
    if (R == 0 && K >= 64 && K <= CONVROT_MAX_K && K % 64 == 0 && pow2_group(group) && K % group == 0)
        return CONVROT_OK;   // empty input: nothing to read or write
    if (!x || !q || !scale) return fail(CONVROT_ERR_NULL, "%s: x, q and scale must be non-NULL", who);
    if (dtype != CONVROT_DTYPE_F32 && dtype != CONVROT_DTYPE_BF16) return fail(CONVROT_ERR_DTYPE, "%s: dtype=%d", who, dtype);
    if (bits != 8 && bits != 4) return fail(CONVROT_ERR_BITS, "%s: bits=%d", who, bits);
    int rc = check_shape(R, 1, K, group, who);
    if (rc) return rc;
    if (bits == 4 && group != 256 && group != 128)
        return fail(CONVROT_ERR_GROUP, "%s: INT4 needs group 256 or 128 (group=%d, K=%lld)", who, group, (long long)K);
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, bits == 8 ? 4 : 2))
        return fail(CONVROT_ERR_ALIGN, "%s: misaligned pointer", who);
    if (R == 0) return CONVROT_OK;
    if ((rc = check_device())) return rc;
    return hip_status(convrot::launch_rotate_quant(x, dtype == CONVROT_DTYPE_F32, R, (int)K, log2i(group), bits, q,
                                                   scale, stream),
                      who);
}

} // namespace

extern "C" {

const char *convrot_status_string(int s)
{
    switch (s) {
    case CONVROT_OK: return "CONVROT_OK";
    case CONVROT_ERR_NULL: return "CONVROT_ERR_NULL";
    case CONVROT_ERR_SHAPE: return "CONVROT_ERR_SHAPE";
    case CONVROT_ERR_GROUP: return "CONVROT_ERR_GROUP";
    case CONVROT_ERR_ALIGN: return "CONVROT_ERR_ALIGN";
    case CONVROT_ERR_DTYPE: return "CONVROT_ERR_DTYPE";
    case CONVROT_ERR_BITS: return "CONVROT_ERR_BITS";
    case CONVROT_ERR_WORKSPACE: return "CONVROT_ERR_WORKSPACE";
    case CONVROT_ERR_HIP: return "CONVROT_ERR_HIP";
    case CONVROT_ERR_DEVICE: return "CONVROT_ERR_DEVICE";
    default: return "CONVROT_ERR_UNKNOWN";
    }
}

const char *convrot_last_error(void) { return g_last_error.c_str(); }

int convrot_dynamic_group(int64_t K, int max_group)
{
    if (K <= 0 || !pow2_group(max_group)) return 0;
    int g = max_group;
    while (K % g) g >>= 1;
    return g;
}

int convrot_prepare_weight(const void *w, int w_dtype, int64_t N, int64_t K, int group, int bits, void *wq,
                           void *w_scale, hipStream_t stream)
{
    return quantize_common(w, w_dtype, N, K, group, bits, wq, w_scale, stream, "convrot_prepare_weight");
}

int convrot_quantize_act(const void *x, int x_dtype, int64_t M, int64_t K, int group, int bits, void *xq,
                         void *x_scale, hipStream_t stream)
{
    return quantize_common(x, x_dtype, M, K, group, bits, xq, x_scale, stream, "convrot_quantize_act");
}

size_t convrot_workspace_bytes(int64_t M, int64_t N, int64_t K, int bits)
{
    // the shapes the entry points accept (check_shape), which also keeps every size below in range
    if (M < 0 || N < 0 || M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31) || K < 64 || K > CONVROT_MAX_K ||
        K % 64 || (bits != 8 && bits != 4))
        return 0;
    return ws_layout(M, N, K, bits).total;
}

} // extern "C"

namespace {

// Shared by convrot_linear (caller's workspace) and convrot_linear_noalloc (the library's fixed
// scratch array).  scratch_fn, when given, is called only after every precondition holds and
// returns the scratch buffer (or sets the status), so a rejected call touches no device.
int linear_i8(const char *who, const void *x, int x_dtype, const int8_t *xq, const float *x_scale, int64_t M,
              int64_t N, int64_t K, int group, const int8_t *wq, const float *w_scale, const float *bias, void *y,
              void *workspace, size_t workspace_bytes, void *(*scratch_fn)(int *), hipStream_t stream)
{
    int rc = check_shape(M, N, K, group, who);
    if (rc) return rc;
    if (M > 16 && (rc = check_gemm_n(N, who))) return rc;
    if (M == 0 || N == 0) return CONVROT_OK;
    if (!wq || !w_scale || !y) return fail(CONVROT_ERR_NULL, "%s: wq, w_scale and y must be non-NULL", who);
    if (!x && (!xq || !x_scale)) return fail(CONVROT_ERR_NULL, "%s: give x, or both xq and x_scale", who);
    if (x && x_dtype != CONVROT_DTYPE_F32 && x_dtype != CONVROT_DTYPE_BF16)
        return fail(CONVROT_ERR_DTYPE, "%s: x_dtype=%d", who, x_dtype);
    if ((x && !aligned(x, 16)) || (!x && (!aligned(xq, 16) || !aligned(x_scale, 4))) || !aligned(wq, 16) ||
        !aligned(w_scale, 4) || !aligned(y, 16) || (bias && !aligned(bias, 4)))
        return fail(CONVROT_ERR_ALIGN, "%s: misaligned pointer", who);
    const WsLayout L = ws_layout(M, N, K, 8);
    if (scratch_fn && x && workspace_bytes < L.part)
        return fail(CONVROT_ERR_WORKSPACE, "%s: M*K = %lld needs %zu bytes of scratch; the fixed scratch holds %zu "
                    "(use convrot_linear with a workspace)", who, (long long)(M * K), L.part, workspace_bytes);
    if (!scratch_fn && x && (!workspace || workspace_bytes < L.part || !aligned(workspace, 256)))
        return fail(CONVROT_ERR_WORKSPACE, "%s: need a 256-byte aligned workspace of at least %zu bytes (got %zu)",
                    who, L.part, workspace ? workspace_bytes : (size_t)0);
    if (M == 0 || N == 0) return CONVROT_OK;
    if ((rc = check_device())) return rc;
    if (scratch_fn) {
        workspace = scratch_fn(&rc);
        if (rc) return rc;
    }

    uint8_t *ws = static_cast<uint8_t *>(workspace);
    // room past the quantized x lets an under-filled GEMM split its tail tiles in K
    void *part = nullptr;
    size_t part_bytes = 0;
    if (M > 16 && ws && aligned(ws, 256) && L.total > L.part && workspace_bytes >= L.total) {
        part = ws + L.part;
        part_bytes = workspace_bytes - L.part;
    }
    if (x) {
        int8_t *qx = reinterpret_cast<int8_t *>(ws + L.xq);
        float *sx = reinterpret_cast<float *>(ws + L.xs);
        rc = hip_status(convrot::launch_rotate_quant(x, x_dtype == CONVROT_DTYPE_F32, M, (int)K, log2i(group), 8, qx,
                                                     sx, stream),
                        "rotate_quant");
        if (rc) return rc;
        xq = qx;
        x_scale = sx;
    }
    hipError_t e = M <= 16 ? convrot::launch_gemv_i8(xq, wq, x_scale, w_scale, bias, y, convrot::Epi::Bf16, M, N,
                                                      (int)K, stream)
                           : convrot::launch_gemm_i8(xq, wq, x_scale, w_scale, bias, y, convrot::Epi::Bf16, M, N,
                                                      (int)K, part, part_bytes, stream);
    return hip_status(e, M <= 16 ? "gemv_i8" : "gemm_i8");
}

// Scratch of convrot_linear_noalloc: one fixed array per GPU, held until the process ends.  On
// the host the array's name is only a stand-in for its device address: the address each device
// holds is looked up once per device (with that device current) and kept in scratch_ptr.
static __device__ __align__(256) uint8_t scratch[CONVROT_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;

void *scratch_for_current_device(int *rc)
{
    static std::mutex mu;
    static void *scratch_ptr[MAX_DEVICES];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        *rc = fail(CONVROT_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
        return nullptr;
    }
    if (dev < 0 || dev >= MAX_DEVICES) {
        *rc = fail(CONVROT_ERR_DEVICE, "device index %d out of range", dev);
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(mu);
    if (!scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            *rc = fail(CONVROT_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
            return nullptr;
        }
        scratch_ptr[dev] = ptr;
    }
    *rc = CONVROT_OK;
    return scratch_ptr[dev];
}

} // namespace

extern "C" {

int convrot_linear(const void *x, int x_dtype, const int8_t *xq, const float *x_scale, int64_t M, int64_t N,
                   int64_t K, int group, const int8_t *wq, const float *w_scale, const float *bias, void *y,
                   void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return linear_i8("convrot_linear", x, x_dtype, xq, x_scale, M, N, K, group, wq, w_scale, bias, y, workspace,
                     workspace_bytes, nullptr, stream);
}

int convrot_linear_noalloc(const void *x, int x_dtype, const int8_t *xq, const float *x_scale, int64_t M, int64_t N,
                           int64_t K, int group, const int8_t *wq, const float *w_scale, const float *bias, void *y,
                           hipStream_t stream)
{
    return linear_i8("convrot_linear_noalloc", x, x_dtype, xq, x_scale, M, N, K, group, wq, w_scale, bias, y, nullptr,
                     CONVROT_NOALLOC_SCRATCH_BYTES, scratch_for_current_device, stream);
}

int convrot_gemm_i8_i32(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K, int32_t *acc,
                        void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    const char *who = "convrot_gemm_i8_i32";
    int rc = check_shape(M, N, K, 1, who);
    if (rc) return rc;
    if (M > 16 && (rc = check_gemm_n(N, who))) return rc;
    if (M == 0 || N == 0) return CONVROT_OK;
    if (!xq || !wq || !acc) return fail(CONVROT_ERR_NULL, "%s: xq, wq and acc must be non-NULL", who);
    if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(acc, 16)) return fail(CONVROT_ERR_ALIGN, "%s: misaligned pointer", who);
    (void)workspace;
    (void)workspace_bytes;
    if ((rc = check_device())) return rc;
    if (M <= 16) {
        return hip_status(convrot::launch_gemv_i8(xq, wq, nullptr, nullptr, nullptr, acc, convrot::Epi::Int32, M, N,
                                                  (int)K, stream),
                          "gemv_i8");
    }
    return hip_status(
        convrot::launch_gemm_i8(xq, wq, nullptr, nullptr, nullptr, acc, convrot::Epi::Int32, M, N, (int)K, nullptr, 0,
                                stream),
        "gemm_i8");
}

} // extern "C"

namespace {

// Shared by convrot_linear_w4a4 (packed INT4 weights, re-encoded on every call) and
// convrot_linear_w4a4_packed (weights re-encoded once by convrot_pack_weight_w4a4).
int linear_w4a4(const char *who, const void *x, int x_dtype, const uint8_t *xq, const uint16_t *x_scale, int64_t M,
                int64_t N, int64_t K, int group, const uint8_t *w, bool w_tiled, const uint16_t *w_scale,
                const float *bias, void *y, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    int rc = check_shape(M, N, K, group, who);
    if (rc) return rc;
    if ((rc = check_gemm_n(N, who))) return rc;
    if ((group != 256 && group != 128) || K % group)
        return fail(CONVROT_ERR_GROUP, "%s: W4A4 needs group 256 or 128 dividing K (group=%d, K=%lld)", who, group,
                    (long long)K);
    if (K < 256) return fail(CONVROT_ERR_SHAPE, "%s: K=%lld; W4A4 needs K >= 256", who, (long long)K);
    if (N % 8) return fail(CONVROT_ERR_SHAPE, "%s: N=%lld must be a multiple of 8", who, (long long)N);
    if (M == 0 || N == 0) return CONVROT_OK;
    if (!w || !w_scale || !y) return fail(CONVROT_ERR_NULL, "%s: the weights, w_scale and y must be non-NULL", who);
    if (!x && (!xq || !x_scale)) return fail(CONVROT_ERR_NULL, "%s: give x, or both xq and x_scale", who);
    if (x && x_dtype != CONVROT_DTYPE_F32 && x_dtype != CONVROT_DTYPE_BF16)
        return fail(CONVROT_ERR_DTYPE, "%s: x_dtype=%d", who, x_dtype);
    if ((x && !aligned(x, 16)) || (!x && (!aligned(xq, 16) || !aligned(x_scale, 2))) || !aligned(w, 16) ||
        !aligned(w_scale, 8) || !aligned(y, 16) || (bias && !aligned(bias, 4)))
        return fail(CONVROT_ERR_ALIGN, "%s: misaligned pointer (w_scale needs 8 bytes)", who);
    const WsLayout L = ws_layout(M, w_tiled ? 0 : N, K, 4);
    if (!workspace || workspace_bytes < L.total || !aligned(workspace, 256))
        return fail(CONVROT_ERR_WORKSPACE, "%s: need a 256-byte aligned workspace of %zu bytes", who, L.total);
    if ((rc = check_device())) return rc;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    if (x) {
        // rotate + quantize straight into the GEMM's FP6 token tiles (no packed INT4 copy)
        rc = hip_status(convrot::launch_rotate_quant_fp6(x, x_dtype == CONVROT_DTYPE_F32, M, (int)K, log2i(group),
                                                         ws + L.tiles, ws + L.xs, stream),
                        "rotate_quant_fp6");
        if (rc) return rc;
        xq = ws + L.tiles;
        x_scale = reinterpret_cast<const uint16_t *>(ws + L.xs);
    }
    return hip_status(convrot::launch_gemm_w4a4(xq, x != nullptr, w, w_tiled, x_scale, w_scale, bias, y,
                                                convrot::Epi::Bf16, M, N, (int)K, group, ws + L.tiles, stream),
                      "gemm_w4a4");
}

} // namespace

extern "C" {

int convrot_linear_w4a4(const void *x, int x_dtype, const uint8_t *xq, const uint16_t *x_scale, int64_t M,
                        int64_t N, int64_t K, int group, const uint8_t *wq, const uint16_t *w_scale,
                        const float *bias, void *y, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return linear_w4a4("convrot_linear_w4a4", x, x_dtype, xq, x_scale, M, N, K, group, wq, false, w_scale, bias, y,
                       workspace, workspace_bytes, stream);
}

size_t convrot_packed_bytes_w4a4(int64_t N, int64_t K)
{
    if (N < 0 || N >= ((int64_t)1 << 31) || K <= 0 || K % 128 || K > CONVROT_MAX_K) return 0;
    return convrot::w4a4_tiled_bytes(0, N, (int)K);
}

int convrot_pack_weight_w4a4(const uint8_t *wq, int64_t N, int64_t K, void *w_packed, hipStream_t stream)
{
    const char *who = "convrot_pack_weight_w4a4";
    int rc = check_shape(N, 1, K, 128, who);
    if (rc) return rc;
    if (K % 128) return fail(CONVROT_ERR_GROUP, "%s: K=%lld must be a multiple of 128", who, (long long)K);
    if (N == 0) return CONVROT_OK;
    if (!wq || !w_packed) return fail(CONVROT_ERR_NULL, "%s: wq and w_packed must be non-NULL", who);
    if (!aligned(wq, 16) || !aligned(w_packed, 16)) return fail(CONVROT_ERR_ALIGN, "%s: misaligned pointer", who);
    if ((rc = check_device())) return rc;
    return hip_status(convrot::launch_tile_w4a4(wq, N, (int)K, static_cast<uint8_t *>(w_packed), stream), "tile_w4a4");
}

int convrot_linear_w4a4_packed(const void *x, int x_dtype, const uint8_t *xq, const uint16_t *x_scale, int64_t M,
                               int64_t N, int64_t K, int group, const void *w_packed, const uint16_t *w_scale,
                               const float *bias, void *y, void *workspace, size_t workspace_bytes,
                               hipStream_t stream)
{
    return linear_w4a4("convrot_linear_w4a4_packed", x, x_dtype, xq, x_scale, M, N, K, group,
                       static_cast<const uint8_t *>(w_packed), true, w_scale, bias, y, workspace, workspace_bytes,
                       stream);
}

size_t convrot_workspace_bytes_w4a8(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || M > CONVROT_W4A8_MAX_M || N < 0 || K <= 0 || K % 128 || K > CONVROT_MAX_K) return 0;
    return ws_layout_w4a8(M, K).total;
}

size_t convrot_packed_bytes_w4a8_group(int64_t N, int64_t K, int group)
{
    if (N < 0 || N >= ((int64_t)1 << 31) || K <= 0 || K > CONVROT_MAX_K || (group != 256 && group != 128) ||
        K % group)
        return 0;
    return convrot::w4a8_packed_bytes(N, (int)K, group);
}

size_t convrot_packed_bytes_w4a8(int64_t N, int64_t K) { return convrot_packed_bytes_w4a8_group(N, K, 256); }

} // extern "C"

namespace {

int pack_w4a8(const char *who, const uint8_t *wq, const uint16_t *w_scale, int64_t N, int64_t K, int group,
              void *w_packed, hipStream_t stream)
{
    int rc = check_shape(N, 1, K, group, who);
    if (rc) return rc;
    if ((group != 256 && group != 128) || K % group)
        return fail(CONVROT_ERR_GROUP, "%s: W4A8 needs group 256 or 128 dividing K (group=%d, K=%lld)", who, group,
                    (long long)K);
    if (N == 0) return CONVROT_OK;
    if (!wq || !w_scale || !w_packed) return fail(CONVROT_ERR_NULL, "%s: wq, w_scale and w_packed must be non-NULL", who);
    if (!aligned(wq, 16) || !aligned(w_scale, 2) || !aligned(w_packed, 16))
        return fail(CONVROT_ERR_ALIGN, "%s: misaligned pointer", who);
    if ((rc = check_device())) return rc;
    return hip_status(
        convrot::launch_pack_w4a8(wq, w_scale, N, (int)K, group, static_cast<uint8_t *>(w_packed), stream),
        "pack_w4a8");
}

} // namespace

extern "C" {

int convrot_pack_weight_w4a8(const uint8_t *wq, const uint16_t *w_scale, int64_t N, int64_t K, void *w_packed,
                             hipStream_t stream)
{
    return pack_w4a8("convrot_pack_weight_w4a8", wq, w_scale, N, K, 256, w_packed, stream);
}

int convrot_pack_weight_w4a8_group(const uint8_t *wq, const uint16_t *w_scale, int64_t N, int64_t K, int group,
                                   void *w_packed, hipStream_t stream)
{
    return pack_w4a8("convrot_pack_weight_w4a8_group", wq, w_scale, N, K, group, w_packed, stream);
}

int convrot_linear_w4a8(const void *x, int x_dtype, const int8_t *xq, const float *x_scale, int64_t M, int64_t N,
                        int64_t K, int group, const void *w_packed, size_t w_packed_bytes, const float *bias, void *y,
                        void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    const char *who = "convrot_linear_w4a8";
    int rc = check_shape(M, N, K, group, who);
    if (rc) return rc;
    if ((group != 256 && group != 128) || K % group)
        return fail(CONVROT_ERR_GROUP, "%s: W4A8 needs group 256 or 128 dividing K (group=%d, K=%lld); the weights "
                    "must be packed with the same group", who, group, (long long)K);
    if (M > CONVROT_W4A8_MAX_M)
        return fail(CONVROT_ERR_SHAPE, "%s: M=%lld tokens; the W4A8 kernel is the decode path (M <= %d)", who,
                    (long long)M, CONVROT_W4A8_MAX_M);
    if (N % 8) return fail(CONVROT_ERR_SHAPE, "%s: N=%lld must be a multiple of 8", who, (long long)N);
    if (M == 0 || N == 0) return CONVROT_OK;
    if (!w_packed || !y) return fail(CONVROT_ERR_NULL, "%s: w_packed and y must be non-NULL", who);
    // the packed size depends on the group (8320 or 8448 bytes per 64 x 256 block): a buffer packed
    // with the other group has another size, and would be read past its end or misread
    const size_t need = convrot_packed_bytes_w4a8_group(N, K, group);
    if (w_packed_bytes != need)
        return fail(CONVROT_ERR_SHAPE, "%s: w_packed_bytes=%zu, but weights packed for N=%lld K=%lld group=%d take %zu "
                    "bytes (were they packed with the other group?)", who, w_packed_bytes, (long long)N, (long long)K,
                    group, need);
    if (!x && (!xq || !x_scale)) return fail(CONVROT_ERR_NULL, "%s: give x, or both xq and x_scale", who);
    if (x && x_dtype != CONVROT_DTYPE_F32 && x_dtype != CONVROT_DTYPE_BF16)
        return fail(CONVROT_ERR_DTYPE, "%s: x_dtype=%d", who, x_dtype);
    if ((x && !aligned(x, 16)) || (!x && (!aligned(xq, 16) || !aligned(x_scale, 4))) || !aligned(w_packed, 16) ||
        !aligned(y, 16) || (bias && !aligned(bias, 4)))
        return fail(CONVROT_ERR_ALIGN, "%s: misaligned pointer", who);
    const WsLayout L = ws_layout_w4a8(M, K);
    if (x && (!workspace || workspace_bytes < L.total || !aligned(workspace, 256)))
        return fail(CONVROT_ERR_WORKSPACE, "%s: need a 256-byte aligned workspace of %zu bytes (got %zu)", who, L.total,
                    workspace ? workspace_bytes : (size_t)0);
    if ((rc = check_device())) return rc;

    uint8_t *ws = static_cast<uint8_t *>(workspace);
    if (x) {
        int8_t *qx = reinterpret_cast<int8_t *>(ws + L.xq);
        float *sx = reinterpret_cast<float *>(ws + L.xs);
        rc = hip_status(convrot::launch_rotate_quant(x, x_dtype == CONVROT_DTYPE_F32, M, (int)K, log2i(group), 8, qx, sx, stream),
                        "rotate_quant");
        if (rc) return rc;
        xq = qx;
        x_scale = sx;
    }
    return hip_status(convrot::launch_gemv_w4a8(xq, x_scale, static_cast<const uint8_t *>(w_packed), bias, y, M, N,
                                                (int)K, group, stream),
                      "gemv_w4a8");
}

int convrot_gemm_i4_i32(const uint8_t *xq, const uint8_t *wq, int64_t M, int64_t N, int64_t K, int32_t *acc,
                        void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    const char *who = "convrot_gemm_i4_i32";
    int rc = check_shape(M, N, K, 256, who);
    if (rc) return rc;
    if ((rc = check_gemm_n(N, who))) return rc;
    if (K % 256 || N % 8) return fail(CONVROT_ERR_SHAPE, "%s: needs K %% 256 == 0 and N %% 8 == 0", who);
    if (M == 0 || N == 0) return CONVROT_OK;
    if (!xq || !wq || !acc) return fail(CONVROT_ERR_NULL, "%s: xq, wq and acc must be non-NULL", who);
    if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(acc, 16)) return fail(CONVROT_ERR_ALIGN, "%s: misaligned pointer", who);
    const WsLayout L = ws_layout(M, N, K, 4);
    if (!workspace || workspace_bytes < L.total || !aligned(workspace, 256))
        return fail(CONVROT_ERR_WORKSPACE, "%s: need a 256-byte aligned workspace of %zu bytes", who, L.total);
    if ((rc = check_device())) return rc;
    return hip_status(convrot::launch_gemm_w4a4(xq, false, wq, false, nullptr, nullptr, nullptr, acc, convrot::Epi::Int32, M, N,
                                                (int)K, 256, static_cast<uint8_t *>(workspace) + L.tiles, stream),
                      "gemm_w4a4");
}

} // extern "C"
