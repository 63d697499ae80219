// C ABI of libgs (include/gs.h): host-side argument validation, scratch
// layout, launch sequencing and error reporting. No C++ exception crosses
// this boundary; no device memory is allocated here.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "gs_internal.h"

// The binning workspace of gs_bin_and_sort_async_noalloc: one fixed array
// per GPU, which each device holds from the library's load on it until the
// process ends. In host code this name is only a stand-in for the symbol;
// its device address on the current device comes from hipGetSymbolAddress
// (static_scratch below), and only that address is ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[GS_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

gs_status fail(gs_status code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

gs_status hip_check(hipError_t e, const char* what) {
    if (e == hipSuccess) return GS_OK;
    return fail(GS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

gs_status check_camera(const gs_camera* cam) {
    if (!cam) return fail(GS_ERR_INVALID, "camera is NULL");
    if (cam->width < 1 || cam->height < 1 || cam->width > GS_MAX_DIM || cam->height > GS_MAX_DIM)
        return fail(GS_ERR_INVALID, "image size %dx%d outside [1, %d]", cam->width, cam->height,
                    GS_MAX_DIM);
    if (!(cam->fx > 0.0f) || !(cam->fy > 0.0f) || !std::isfinite(cam->fx) || !std::isfinite(cam->fy))
        return fail(GS_ERR_INVALID, "focal lengths must be finite and positive");
    if (!std::isfinite(cam->cx) || !std::isfinite(cam->cy))
        return fail(GS_ERR_INVALID, "principal point must be finite");
    for (int i = 0; i < 9; ++i)
        if (!std::isfinite(cam->R[i])) return fail(GS_ERR_INVALID, "R must be finite");
    for (int i = 0; i < 3; ++i)
        if (!std::isfinite(cam->t[i]) || !std::isfinite(cam->campos[i]))
            return fail(GS_ERR_INVALID, "t and campos must be finite");
    return GS_OK;
}

}  // namespace

extern "C" {

void gs_constants(float out[9]) {
    out[0] = (float)gs::kTile;
    out[1] = gs::kDilation;
    out[2] = gs::kZNear;
    out[3] = gs::kFrustumClamp;
    out[4] = gs::kDiscFloor;
    out[5] = gs::kSigma;
    out[6] = gs::kAlphaMin;
    out[7] = gs::kAlphaMax;
    out[8] = gs::kTStop;
}

const char* gs_last_error(void) { return g_last_error.c_str(); }

void gs_version(int32_t out[3]) {
    out[0] = 0;
    out[1] = 1;
    out[2] = 0;
}

gs_status gs_preprocess_ex(const gs_camera* cam, int32_t n, const float* means, const float* scales,
                           const float* quats, const float* opacity, const float* sh,
                           int32_t sh_degree, const float* rgb_in, float* xy_depth, float* conic_op,
                           float* rgb, uint32_t* tiles_touched, uint32_t flags, void* stream) {
    g_last_error.clear();
    if (gs_status s = check_camera(cam)) return s;
    if (flags & ~(uint32_t)GS_TILES_ELLIPSE) return fail(GS_ERR_INVALID, "unknown flags 0x%x", flags);
    if (n < 0 || n > GS_MAX_GAUSSIANS) return fail(GS_ERR_INVALID, "n = %d outside [0, %d]", n, GS_MAX_GAUSSIANS);
    if (n == 0) return GS_OK;
    if (!means || !scales || !quats || !opacity || !xy_depth || !conic_op || !rgb || !tiles_touched)
        return fail(GS_ERR_INVALID, "gs_preprocess: a required pointer is NULL");
    if (sh) {
        if (sh_degree < 0 || sh_degree > 3) return fail(GS_ERR_INVALID, "sh_degree %d outside 0..3", sh_degree);
    } else if (!rgb_in) {
        return fail(GS_ERR_INVALID, "gs_preprocess: rgb_in is required when sh is NULL");
    }
    if (((uintptr_t)xy_depth | (uintptr_t)conic_op | (uintptr_t)rgb) & 15)
        return fail(GS_ERR_INVALID, "gs_preprocess: float4 outputs must be 16-byte aligned");
    return hip_check(gs::launch_preprocess(*cam, n, means, scales, quats, opacity, sh, sh_degree,
                                           rgb_in, (float4*)xy_depth, (float4*)conic_op,
                                           (float4*)rgb, tiles_touched, flags, (hipStream_t)stream),
                     "gs_preprocess launch");
}

gs_status gs_preprocess(const gs_camera* cam, int32_t n, const float* means, const float* scales,
                        const float* quats, const float* opacity, const float* sh,
                        int32_t sh_degree, const float* rgb_in, float* xy_depth, float* conic_op,
                        float* rgb, uint32_t* tiles_touched, void* stream) {
    return gs_preprocess_ex(cam, n, means, scales, quats, opacity, sh, sh_degree, rgb_in, xy_depth, conic_op,
                            rgb, tiles_touched, GS_TILES_SQUARE, stream);
}

gs_status gs_preprocess_views(const gs_camera* cams, int32_t n_views, int32_t n, const float* means,
                              const float* scales, const float* quats, const float* opacity, const float* sh,
                              int32_t sh_degree, const float* rgb_in, float* xy_depth, float* conic_op, float* rgb,
                              uint32_t* tiles_touched, uint32_t flags, void* stream) {
    g_last_error.clear();
    if (!cams) return fail(GS_ERR_INVALID, "gs_preprocess_views: cams is NULL");
    if (n_views < 1 || n_views > GS_MAX_VIEWS)
        return fail(GS_ERR_INVALID, "gs_preprocess_views: n_views = %d outside [1, %d]", n_views, GS_MAX_VIEWS);
    gs::CameraSet set{};
    set.n = n_views;
    for (int v = 0; v < n_views; ++v) {
        if (gs_status s = check_camera(&cams[v])) return s;
        if (cams[v].width != cams[0].width || cams[v].height != cams[0].height)
            return fail(GS_ERR_INVALID, "gs_preprocess_views: camera %d is not %dx%d like camera 0", v,
                        cams[0].width, cams[0].height);
        set.cam[v] = cams[v];
    }
    if (n < 0 || (int64_t)n * n_views > GS_MAX_GAUSSIANS)
        return fail(GS_ERR_INVALID, "n = %d (x %d views) outside [0, %d]", n, n_views, GS_MAX_GAUSSIANS);
    if (sh && (sh_degree < 0 || sh_degree > 3))
        return fail(GS_ERR_INVALID, "sh_degree %d outside [0, 3]", sh_degree);
    if (flags & ~(uint32_t)GS_TILES_ELLIPSE) return fail(GS_ERR_INVALID, "gs_preprocess_views: unknown flags");
    if (n == 0) return GS_OK;
    if (!means || !scales || !quats || !opacity || (!sh && !rgb_in) || !xy_depth || !conic_op || !rgb ||
        !tiles_touched)
        return fail(GS_ERR_INVALID, "gs_preprocess_views: a required pointer is NULL");
    if (((uintptr_t)xy_depth | (uintptr_t)conic_op | (uintptr_t)rgb) & 15)
        return fail(GS_ERR_INVALID, "gs_preprocess_views: float4 outputs must be 16-byte aligned");
    return hip_check(gs::launch_preprocess_views(set, n, means, scales, quats, opacity, sh, sh_degree, rgb_in,
                                                 (float4*)xy_depth, (float4*)conic_op, (float4*)rgb, tiles_touched,
                                                 flags, (hipStream_t)stream),
                     "gs_preprocess_views launch");
}

gs_status gs_preprocess_bwd(const gs_camera* cam, int32_t n, const float* means, const float* scales,
                            const float* quats, const float* sh, int32_t sh_degree,
                            const uint32_t* tiles_touched, const float* grad_mean2d,
                            const float* grad_conic_op, const float* grad_rgb, float* grad_means,
                            float* grad_scales, float* grad_quats, float* grad_opacity, float* grad_sh,
                            float* grad_rgb_in, void* stream) {
    g_last_error.clear();
    if (gs_status s = check_camera(cam)) return s;
    if (n < 0 || n > GS_MAX_GAUSSIANS) return fail(GS_ERR_INVALID, "n = %d outside [0, %d]", n, GS_MAX_GAUSSIANS);
    if (n == 0) return GS_OK;
    if (!means || !scales || !quats || !tiles_touched || !grad_mean2d || !grad_conic_op || !grad_rgb ||
        !grad_means || !grad_scales || !grad_quats || !grad_opacity)
        return fail(GS_ERR_INVALID, "gs_preprocess_bwd: a required pointer is NULL");
    if (sh) {
        if (sh_degree < 0 || sh_degree > 3) return fail(GS_ERR_INVALID, "sh_degree %d outside 0..3", sh_degree);
        if (!grad_sh) return fail(GS_ERR_INVALID, "gs_preprocess_bwd: grad_sh is required when sh is given");
    } else if (!grad_rgb_in) {
        return fail(GS_ERR_INVALID, "gs_preprocess_bwd: grad_rgb_in is required when sh is NULL");
    }
    if (((uintptr_t)grad_conic_op | (uintptr_t)grad_rgb) & 15)
        return fail(GS_ERR_INVALID, "gs_preprocess_bwd: float4 gradients must be 16-byte aligned");
    if ((uintptr_t)grad_mean2d & 7)
        return fail(GS_ERR_INVALID, "gs_preprocess_bwd: grad_mean2d must be 8-byte aligned");
    return hip_check(gs::launch_preprocess_bwd(*cam, n, means, scales, quats, sh, sh_degree, tiles_touched,
                                               (const float2*)grad_mean2d, (const float4*)grad_conic_op,
                                               (const float4*)grad_rgb, grad_means, grad_scales, grad_quats,
                                               grad_opacity, sh ? grad_sh : nullptr, sh ? nullptr : grad_rgb_in,
                                               (hipStream_t)stream),
                     "gs_preprocess_bwd launch");
}

namespace {

// Checks shared by the blocking and the asynchronous binning entry points;
// on GS_OK with scratch != NULL, *s is laid out in scratch.
gs_status bin_args(const char* fn, const gs_camera* cam, int32_t n, const float* xy_depth,
                   const uint32_t* tiles_touched, const uint64_t* keys, const uint32_t* point_list,
                   int64_t capacity, void* scratch, size_t* scratch_bytes, bool* size_query, gs::BinScratch* s,
                   int32_t n_views = 1) {
    if (gs_status st = check_camera(cam)) return st;
    if (n_views < 1 || n_views > GS_MAX_VIEWS)
        return fail(GS_ERR_INVALID, "%s: n_views = %d outside [1, %d]", fn, n_views, GS_MAX_VIEWS);
    if (n < 0 || (int64_t)n * n_views > GS_MAX_GAUSSIANS)
        return fail(GS_ERR_INVALID, "n = %d (x %d views) outside [0, %d]", n, n_views, GS_MAX_GAUSSIANS);
    if ((int64_t)gs::tiles_x(*cam) * gs::tiles_y(*cam) * n_views > (1 << 24))
        return fail(GS_ERR_INVALID, "%s: more than 2^24 tiles", fn);
    n *= n_views;
    if (capacity < 0 || capacity > (int64_t)UINT32_MAX)
        return fail(GS_ERR_INVALID, "capacity %lld outside [0, 2^32 - 1]", (long long)capacity);
    if (!scratch_bytes) return fail(GS_ERR_INVALID, "%s: scratch_bytes is NULL", fn);
    const size_t need = gs::bin_scratch_layout(n, capacity, nullptr, nullptr);
    *size_query = scratch == nullptr;
    if (*size_query) {
        *scratch_bytes = need;
        return GS_OK;
    }
    if (*scratch_bytes < need)
        return fail(GS_ERR_INVALID, "%s: scratch of %zu bytes is smaller than the %zu required", fn,
                    *scratch_bytes, need);
    if ((uintptr_t)scratch & 255) return fail(GS_ERR_INVALID, "%s: scratch must be 256-byte aligned", fn);
    if (n > 0 && (!xy_depth || !tiles_touched || (capacity > 0 && (!keys || !point_list))))
        return fail(GS_ERR_INVALID, "%s: a required pointer is NULL", fn);
    if (n > 0 && ((uintptr_t)xy_depth & 15)) return fail(GS_ERR_INVALID, "%s: xy_depth must be 16-byte aligned", fn);
    gs::bin_scratch_layout(n, capacity, s, scratch);
    return GS_OK;
}

// The tile-test flags of the binning entry points: the ellipse test reads
// the conic of every splat.
gs_status tile_test_args(const char* fn, int32_t n, const float* conic_op, uint32_t flags) {
    if (flags & ~(uint32_t)GS_TILES_ELLIPSE) return fail(GS_ERR_INVALID, "%s: unknown flags 0x%x", fn, flags);
    if ((flags & GS_TILES_ELLIPSE) && n > 0 && (!conic_op || ((uintptr_t)conic_op & 15)))
        return fail(GS_ERR_INVALID, "%s: the ellipse test needs a 16-byte aligned conic_op", fn);
    return GS_OK;
}

}  // namespace

gs_status gs_bin_and_sort_ex(const gs_camera* cam, int32_t n, const float* xy_depth, const float* conic_op,
                             const uint32_t* tiles_touched, uint64_t* keys, uint32_t* point_list,
                             int64_t capacity, void* scratch, size_t* scratch_bytes, int64_t* n_entries,
                             uint32_t flags, void* stream) {
    g_last_error.clear();
    gs::BinScratch s{};
    bool query = false;
    if (gs_status e = bin_args("gs_bin_and_sort", cam, n, xy_depth, tiles_touched, keys, point_list, capacity,
                               scratch, scratch_bytes, &query, &s))
        return e;
    if (query) return GS_OK;
    if (gs_status e = tile_test_args("gs_bin_and_sort", n, conic_op, flags)) return e;
    if (!n_entries) return fail(GS_ERR_INVALID, "gs_bin_and_sort: n_entries is NULL");
    *n_entries = 0;
    if (n == 0) return GS_OK;
    hipStream_t st = (hipStream_t)stream;
    if (gs_status e = hip_check(gs::launch_bin_and_sort(*cam, 1, n, (const float4*)xy_depth, (const float4*)conic_op,
                                                        tiles_touched, keys, point_list, (uint32_t)capacity, s,
                                                        nullptr, flags, st),
                                "bin_and_sort launch"))
        return e;
    // the entry count, once everything is enqueued
    uint64_t total = 0;
    if (gs_status e = hip_check(hipMemcpyAsync(&total, s.total, sizeof(total), hipMemcpyDeviceToHost, st),
                                "entry count copy"))
        return e;
    if (gs_status e = hip_check(hipStreamSynchronize(st), "entry count sync")) return e;
    *n_entries = (int64_t)total;
    if (total > (uint64_t)UINT32_MAX)
        return fail(GS_ERR_OVERFLOW, "%llu entries do not fit in 32 bits", (unsigned long long)total);
    if ((int64_t)total > capacity)
        return fail(GS_ERR_CAPACITY, "%llu entries exceed the capacity %lld", (unsigned long long)total,
                    (long long)capacity);
    return GS_OK;
}

gs_status gs_bin_and_sort(const gs_camera* cam, int32_t n, const float* xy_depth,
                          const uint32_t* tiles_touched, uint64_t* keys, uint32_t* point_list,
                          int64_t capacity, void* scratch, size_t* scratch_bytes,
                          int64_t* n_entries, void* stream) {
    return gs_bin_and_sort_ex(cam, n, xy_depth, nullptr, tiles_touched, keys, point_list, capacity, scratch,
                              scratch_bytes, n_entries, GS_TILES_SQUARE, stream);
}

gs_status gs_bin_and_sort_views_async(const gs_camera* cam, int32_t n_views, int32_t n, const float* xy_depth,
                                      const float* conic_op, const uint32_t* tiles_touched, uint64_t* keys,
                                      uint32_t* point_list, int64_t capacity, void* scratch, size_t* scratch_bytes,
                                      uint64_t* n_entries_dev, uint32_t flags, void* stream) {
    g_last_error.clear();
    gs::BinScratch s{};
    bool query = false;
    if (gs_status e = bin_args("gs_bin_and_sort_async", cam, n, xy_depth, tiles_touched, keys, point_list,
                               capacity, scratch, scratch_bytes, &query, &s, n_views))
        return e;
    if (query) return GS_OK;
    const int32_t n_all = n * n_views;
    if (gs_status e = tile_test_args("gs_bin_and_sort_async", n_all, conic_op, flags)) return e;
    if (!n_entries_dev || ((uintptr_t)n_entries_dev & 7))
        return fail(GS_ERR_INVALID, "gs_bin_and_sort_async: n_entries_dev must be an 8-byte aligned device pointer");
    hipStream_t st = (hipStream_t)stream;
    if (n_all == 0)
        return hip_check(gs::launch_fill_u32((uint32_t*)n_entries_dev, 2, 0u, st), "entry count clear");
    return hip_check(gs::launch_bin_and_sort(*cam, n_views, n_all, (const float4*)xy_depth, (const float4*)conic_op,
                                             tiles_touched, keys, point_list, (uint32_t)capacity, s, n_entries_dev,
                                             flags, st),
                     "bin_and_sort launch");
}

gs_status gs_bin_and_sort_async_ex(const gs_camera* cam, int32_t n, const float* xy_depth, const float* conic_op,
                                   const uint32_t* tiles_touched, uint64_t* keys, uint32_t* point_list,
                                   int64_t capacity, void* scratch, size_t* scratch_bytes,
                                   uint64_t* n_entries_dev, uint32_t flags, void* stream) {
    return gs_bin_and_sort_views_async(cam, 1, n, xy_depth, conic_op, tiles_touched, keys, point_list, capacity,
                                       scratch, scratch_bytes, n_entries_dev, flags, stream);
}

gs_status gs_bin_and_sort_async(const gs_camera* cam, int32_t n, const float* xy_depth,
                                const uint32_t* tiles_touched, uint64_t* keys, uint32_t* point_list,
                                int64_t capacity, void* scratch, size_t* scratch_bytes,
                                uint64_t* n_entries_dev, void* stream) {
    return gs_bin_and_sort_async_ex(cam, n, xy_depth, nullptr, tiles_touched, keys, point_list, capacity,
                                    scratch, scratch_bytes, n_entries_dev, GS_TILES_SQUARE, stream);
}

}  // extern "C"

namespace {

// Device address of `scratch` on each device, looked up on the first
// no-allocation call made with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices] = {};

gs_status static_scratch(void** out) {
    int dev = -1;
    if (gs_status e = hip_check(hipGetDevice(&dev), "hipGetDevice")) return e;
    if (dev < 0 || dev >= kMaxDevices) return fail(GS_ERR_INVALID, "device %d outside [0, %d)", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_static_mu);
    if (!g_static_ptr[dev]) {
        void* p = nullptr;
        if (gs_status e = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"))
            return e;
        if (!p || ((uintptr_t)p & 255)) return fail(GS_ERR_HIP, "static workspace has no 256-byte aligned address");
        g_static_ptr[dev] = p;
    }
    *out = g_static_ptr[dev];
    return GS_OK;
}

}  // namespace

extern "C" {

gs_status gs_bin_and_sort_async_noalloc(const gs_camera* cam, int32_t n, const float* xy_depth,
                                        const float* conic_op, const uint32_t* tiles_touched, uint64_t* keys,
                                        uint32_t* point_list, int64_t capacity, uint64_t* n_entries_dev,
                                        uint32_t flags, void* stream) {
    g_last_error.clear();
    const char* fn = "gs_bin_and_sort_async_noalloc";
    gs::BinScratch s{};
    bool query = false;
    size_t need = 0;
    // the size first (no device call): arguments and the workspace this call needs
    if (gs_status e = bin_args(fn, cam, n, xy_depth, tiles_touched, keys, point_list, capacity, nullptr, &need,
                               &query, &s))
        return e;
    if (need > (size_t)GS_NOALLOC_SCRATCH_BYTES)
        return fail(GS_ERR_INVALID,
                    "%s: n = %d and capacity = %lld need %zu bytes of workspace, more than the fixed %zu; "
                    "use gs_bin_and_sort_async_ex with a caller-owned workspace",
                    fn, n, (long long)capacity, need, (size_t)GS_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (gs_status e = static_scratch(&ws)) return e;
    size_t have = GS_NOALLOC_SCRATCH_BYTES;
    if (gs_status e = bin_args(fn, cam, n, xy_depth, tiles_touched, keys, point_list, capacity, ws, &have, &query,
                               &s))
        return e;
    if (gs_status e = tile_test_args(fn, n, conic_op, flags)) return e;
    if (!n_entries_dev || ((uintptr_t)n_entries_dev & 7))
        return fail(GS_ERR_INVALID, "%s: n_entries_dev must be an 8-byte aligned device pointer", fn);
    hipStream_t st = (hipStream_t)stream;
    if (n == 0) return hip_check(gs::launch_fill_u32((uint32_t*)n_entries_dev, 2, 0u, st), "entry count clear");
    return hip_check(gs::launch_bin_and_sort(*cam, 1, n, (const float4*)xy_depth, (const float4*)conic_op,
                                             tiles_touched, keys, point_list, (uint32_t)capacity, s, n_entries_dev,
                                             flags, st),
                     "bin_and_sort launch");
}

namespace {

gs_status appearance_args(const char* fn, const gs_camera* cam, int32_t n, int32_t L, int32_t H) {
    if (gs_status s = check_camera(cam)) return s;
    if (n < 0 || n > GS_MAX_GAUSSIANS) return fail(GS_ERR_INVALID, "%s: n = %d outside [0, %d]", fn, n, GS_MAX_GAUSSIANS);
    if (L < 1 || L > GS_APP_MAX_LATENT) return fail(GS_ERR_INVALID, "%s: n_latent %d outside [1, %d]", fn, L, GS_APP_MAX_LATENT);
    if (H < 1 || H > GS_APP_MAX_HIDDEN) return fail(GS_ERR_INVALID, "%s: n_hidden %d outside [1, %d]", fn, H, GS_APP_MAX_HIDDEN);
    return GS_OK;
}

}  // namespace

gs_status gs_appearance_fwd(const gs_camera* cam, int32_t n, const float* means, const float* latent,
                            int32_t n_latent, int32_t n_hidden, const float* weights, float* rgb, void* stream) {
    g_last_error.clear();
    if (gs_status s = appearance_args("gs_appearance_fwd", cam, n, n_latent, n_hidden)) return s;
    if (n == 0) return GS_OK;
    if (!means || !latent || !weights || !rgb) return fail(GS_ERR_INVALID, "gs_appearance_fwd: a required pointer is NULL");
    return hip_check(gs::launch_appearance_fwd(*cam, n, means, latent, n_latent, n_hidden, weights, rgb,
                                               (hipStream_t)stream),
                     "gs_appearance_fwd launch");
}

gs_status gs_appearance_bwd(const gs_camera* cam, int32_t n, const float* means, const float* latent,
                            int32_t n_latent, int32_t n_hidden, const float* weights, const float* grad_rgb,
                            float* grad_latent, float* grad_weights, void* scratch, size_t* scratch_bytes,
                            void* stream) {
    g_last_error.clear();
    if (gs_status s = appearance_args("gs_appearance_bwd", cam, n, n_latent, n_hidden)) return s;
    if (!scratch_bytes) return fail(GS_ERR_INVALID, "gs_appearance_bwd: scratch_bytes is NULL");
    const size_t need = gs::appearance_bwd_scratch(n, n_latent, n_hidden);
    if (!scratch) {
        *scratch_bytes = need;
        return GS_OK;
    }
    if (*scratch_bytes < need)
        return fail(GS_ERR_INVALID, "gs_appearance_bwd: scratch of %zu bytes is smaller than the %zu required",
                    *scratch_bytes, need);
    if ((uintptr_t)scratch & 3) return fail(GS_ERR_INVALID, "gs_appearance_bwd: scratch must be 4-byte aligned");
    if (!grad_weights || (n > 0 && (!means || !latent || !weights || !grad_rgb || !grad_latent)))
        return fail(GS_ERR_INVALID, "gs_appearance_bwd: a required pointer is NULL");
    return hip_check(gs::launch_appearance_bwd(*cam, n, means, latent, n_latent, n_hidden, weights, grad_rgb,
                                               grad_latent, grad_weights, (float*)scratch, (hipStream_t)stream),
                     "gs_appearance_bwd launch");
}

gs_status gs_tile_ranges(const gs_camera* cam, const uint64_t* keys, int64_t n_entries,
                         uint32_t* ranges, uint32_t* tile_order, void* stream) {
    g_last_error.clear();
    if (gs_status s = check_camera(cam)) return s;
    if (n_entries < 0 || n_entries > (int64_t)UINT32_MAX)
        return fail(GS_ERR_INVALID, "n_entries %lld outside [0, 2^32 - 1]", (long long)n_entries);
    if (!ranges || (n_entries > 0 && !keys)) return fail(GS_ERR_INVALID, "gs_tile_ranges: NULL pointer");
    const int n_tiles = gs::tiles_x(*cam) * gs::tiles_y(*cam);
    return hip_check(gs::launch_tile_ranges(keys, (uint32_t)n_entries, nullptr, 0u, n_tiles, ranges, tile_order,
                                            nullptr, (hipStream_t)stream),
                     "tile ranges launch");
}

gs_status gs_tile_ranges_async(const gs_camera* cam, const uint64_t* keys, const uint64_t* n_entries_dev,
                               int64_t capacity, uint32_t* ranges, uint32_t* tile_order, void* stream) {
    g_last_error.clear();
    if (gs_status s = check_camera(cam)) return s;
    if (capacity < 0 || capacity > (int64_t)UINT32_MAX)
        return fail(GS_ERR_INVALID, "capacity %lld outside [0, 2^32 - 1]", (long long)capacity);
    if (!ranges || !n_entries_dev || ((uintptr_t)n_entries_dev & 7) || (capacity > 0 && !keys))
        return fail(GS_ERR_INVALID, "gs_tile_ranges_async: NULL or misaligned pointer");
    const int n_tiles = gs::tiles_x(*cam) * gs::tiles_y(*cam);
    return hip_check(gs::launch_tile_ranges(keys, 0u, n_entries_dev, (uint32_t)capacity, n_tiles, ranges,
                                            tile_order, nullptr, (hipStream_t)stream),
                     "tile ranges launch");
}

gs_status gs_tile_ranges_ex(const gs_camera* cam, int32_t n_views, const uint64_t* keys, int64_t n_entries,
                            const uint64_t* n_entries_dev, int64_t capacity, uint32_t* ranges,
                            uint32_t* tile_order, uint32_t* chunks, void* stream) {
    g_last_error.clear();
    if (gs_status s = check_camera(cam)) return s;
    if (n_views < 1 || n_views > GS_MAX_VIEWS)
        return fail(GS_ERR_INVALID, "gs_tile_ranges_ex: n_views = %d outside [1, %d]", n_views, GS_MAX_VIEWS);
    if (capacity < 0 || capacity > (int64_t)UINT32_MAX)
        return fail(GS_ERR_INVALID, "capacity %lld outside [0, 2^32 - 1]", (long long)capacity);
    if (!n_entries_dev && (n_entries < 0 || n_entries > capacity))
        return fail(GS_ERR_INVALID, "n_entries %lld outside [0, capacity %lld]", (long long)n_entries,
                    (long long)capacity);
    if (!ranges || (capacity > 0 && !keys) || ((uintptr_t)n_entries_dev & 7) || ((uintptr_t)chunks & 15))
        return fail(GS_ERR_INVALID, "gs_tile_ranges_ex: NULL or misaligned pointer");
    const int n_tiles = gs::tiles_x(*cam) * gs::tiles_y(*cam) * n_views;
    return hip_check(gs::launch_tile_ranges(keys, n_entries_dev ? 0u : (uint32_t)n_entries, n_entries_dev,
                                            (uint32_t)capacity, n_tiles, ranges, tile_order, chunks,
                                            (hipStream_t)stream),
                     "tile ranges launch");
}

gs_status gs_composite_fwd(const gs_camera* cam, const uint32_t* ranges, const uint32_t* point_list,
                           const float* xy_depth, const float* conic_op, const float* rgb,
                           const float bg[3], float* image, float* final_T, uint32_t* n_contrib,
                           uint32_t* n_examined, const uint32_t* tile_order, void* stream) {
    g_last_error.clear();
    if (gs_status s = check_camera(cam)) return s;
    if (!ranges || !bg || !image || !final_T || !n_contrib)
        return fail(GS_ERR_INVALID, "gs_composite_fwd: a required pointer is NULL");
    if (((uintptr_t)xy_depth | (uintptr_t)conic_op | (uintptr_t)rgb) & 15)
        return fail(GS_ERR_INVALID, "gs_composite_fwd: float4 inputs must be 16-byte aligned");
    const float3 b = make_float3(bg[0], bg[1], bg[2]);
    return hip_check(gs::launch_composite_fwd(*cam, 1, ranges, point_list, (const float4*)xy_depth,
                                              (const float4*)conic_op, (const float4*)rgb, b, image,
                                              final_T, n_contrib, n_examined, tile_order, nullptr, 0u,
                                              nullptr, nullptr, (hipStream_t)stream),
                     "composite fwd launch");
}

gs_status gs_composite_fwd_ex(const gs_camera* cam, int32_t n_views, const uint32_t* ranges,
                              const uint32_t* point_list, const float* xy_depth, const float* conic_op,
                              const float* rgb, const float bg[3], float* image, float* final_T, uint32_t* n_contrib,
                              uint32_t* n_examined, const uint32_t* tile_order, int64_t capacity,
                              float* ckpt, const uint32_t* chunks, void* part, void* stream) {
    g_last_error.clear();
    if (n_views < 1 || n_views > GS_MAX_VIEWS)
        return fail(GS_ERR_INVALID, "gs_composite_fwd_ex: n_views = %d outside [1, %d]", n_views, GS_MAX_VIEWS);
    if (!ckpt && !chunks && n_views == 1)
        return gs_composite_fwd(cam, ranges, point_list, xy_depth, conic_op, rgb, bg, image, final_T, n_contrib,
                                n_examined, tile_order, stream);
    if (gs_status s = check_camera(cam)) return s;
    if (capacity < 0 || capacity > (int64_t)UINT32_MAX)
        return fail(GS_ERR_INVALID, "gs_composite_fwd_ex: capacity %lld outside [0, 2^32 - 1]", (long long)capacity);
    if (!bg || !image || !final_T || !n_contrib || (!chunks && !ranges))
        return fail(GS_ERR_INVALID, "gs_composite_fwd_ex: a required pointer is NULL");
    if (chunks && !part) return fail(GS_ERR_INVALID, "gs_composite_fwd_ex: chunks without the part workspace");
    if (((uintptr_t)xy_depth | (uintptr_t)conic_op | (uintptr_t)rgb | (uintptr_t)ckpt | (uintptr_t)chunks |
         (uintptr_t)part) & 15)
        return fail(GS_ERR_INVALID, "gs_composite_fwd_ex: float4 buffers must be 16-byte aligned");
    const float3 b = make_float3(bg[0], bg[1], bg[2]);
    return hip_check(gs::launch_composite_fwd(*cam, n_views, ranges, point_list, (const float4*)xy_depth,
                                              (const float4*)conic_op, (const float4*)rgb, b, image,
                                              final_T, n_contrib, n_examined, tile_order, (float4*)ckpt,
                                              (uint32_t)capacity, chunks, part, (hipStream_t)stream),
                     "composite fwd launch");
}

size_t gs_composite_part_bytes(const gs_camera* cam, int32_t n_views, int64_t capacity) {
    if (!cam || check_camera(cam) != GS_OK || capacity < 0 || capacity > (int64_t)UINT32_MAX) return 0;
    if (n_views < 1 || n_views > GS_MAX_VIEWS) return 0;
    return gs::composite_part_bytes(*cam, n_views, (uint32_t)capacity);
}

gs_status gs_composite_bwd(const gs_camera* cam, int32_t n, const uint32_t* ranges,
                           const uint32_t* point_list, const float* xy_depth,
                           const float* conic_op, const float* rgb, const float bg[3],
                           const float* final_T, const uint32_t* n_contrib,
                           const float* dL_dimage, float* grad_mean2d, float* grad_conic_op,
                           float* grad_rgb, const uint32_t* tile_order, void* stream) {
    g_last_error.clear();
    if (gs_status s = check_camera(cam)) return s;
    if (n < 0 || n > GS_MAX_GAUSSIANS) return fail(GS_ERR_INVALID, "n = %d outside [0, %d]", n, GS_MAX_GAUSSIANS);
    if (!ranges || !bg || !final_T || !n_contrib || !dL_dimage)
        return fail(GS_ERR_INVALID, "gs_composite_bwd: a required pointer is NULL");
    if (n > 0 && (!grad_mean2d || !grad_conic_op || !grad_rgb))
        return fail(GS_ERR_INVALID, "gs_composite_bwd: a gradient pointer is NULL");
    if (((uintptr_t)xy_depth | (uintptr_t)conic_op | (uintptr_t)rgb | (uintptr_t)grad_conic_op |
         (uintptr_t)grad_rgb) & 15 || ((uintptr_t)grad_mean2d & 7))
        return fail(GS_ERR_INVALID, "gs_composite_bwd: misaligned vector buffer");
    const float3 b = make_float3(bg[0], bg[1], bg[2]);
    return hip_check(gs::launch_composite_bwd(*cam, 1, n, ranges, point_list, (const float4*)xy_depth,
                                              (const float4*)conic_op, (const float4*)rgb, b, final_T,
                                              n_contrib, dL_dimage, (float2*)grad_mean2d,
                                              (float4*)grad_conic_op, (float4*)grad_rgb, tile_order,
                                              nullptr, 0u, nullptr, nullptr, (hipStream_t)stream),
                     "composite bwd launch");
}

gs_status gs_composite_bwd_ex(const gs_camera* cam, int32_t n_views, int32_t n, const uint32_t* ranges,
                              const uint32_t* point_list, const uint32_t* chunks, int64_t capacity,
                              const float* xy_depth, const float* conic_op, const float* rgb,
                              const float bg[3], const float* image, const float* final_T,
                              const uint32_t* n_contrib, const float* ckpt, const float* dL_dimage,
                              float* grad_mean2d, float* grad_conic_op, float* grad_rgb, void* stream) {
    g_last_error.clear();
    if (gs_status s = check_camera(cam)) return s;
    if (n_views < 1 || n_views > GS_MAX_VIEWS)
        return fail(GS_ERR_INVALID, "gs_composite_bwd_ex: n_views = %d outside [1, %d]", n_views, GS_MAX_VIEWS);
    if (n < 0 || n > GS_MAX_GAUSSIANS) return fail(GS_ERR_INVALID, "n = %d outside [0, %d]", n, GS_MAX_GAUSSIANS);
    if (capacity < 0 || capacity > (int64_t)UINT32_MAX)
        return fail(GS_ERR_INVALID, "gs_composite_bwd_ex: capacity %lld outside [0, 2^32 - 1]", (long long)capacity);
    if (!ranges || !bg || !final_T || !n_contrib || !dL_dimage || !image || !chunks)
        return fail(GS_ERR_INVALID, "gs_composite_bwd_ex: a required pointer is NULL");
    if (capacity > 0 && !ckpt) return fail(GS_ERR_INVALID, "gs_composite_bwd_ex: ckpt is NULL");
    if (n > 0 && (!grad_mean2d || !grad_conic_op || !grad_rgb))
        return fail(GS_ERR_INVALID, "gs_composite_bwd_ex: a gradient pointer is NULL");
    if (((uintptr_t)xy_depth | (uintptr_t)conic_op | (uintptr_t)rgb | (uintptr_t)grad_conic_op |
         (uintptr_t)grad_rgb | (uintptr_t)ckpt | (uintptr_t)chunks) & 15 || ((uintptr_t)grad_mean2d & 7))
        return fail(GS_ERR_INVALID, "gs_composite_bwd_ex: misaligned vector buffer");
    const float3 b = make_float3(bg[0], bg[1], bg[2]);
    return hip_check(gs::launch_composite_bwd(*cam, n_views, n, ranges, point_list, (const float4*)xy_depth,
                                              (const float4*)conic_op, (const float4*)rgb, b, final_T,
                                              n_contrib, dL_dimage, (float2*)grad_mean2d,
                                              (float4*)grad_conic_op, (float4*)grad_rgb, nullptr, chunks,
                                              (uint32_t)capacity, (const float4*)ckpt, image, (hipStream_t)stream),
                     "composite bwd launch");
}

}  // extern "C"
