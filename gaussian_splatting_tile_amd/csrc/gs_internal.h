// Internal declarations shared by the libgs translation units (kernels and
// the C-ABI layer). Not installed; the public interface is include/gs.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gs.h"

namespace gs {

// Method constants. learn-gs constants block (TILE, DILATION, ALPHA_MIN,
// ALPHA_MAX, T_STOP, Z_NEAR); "rigel" README "Projection" (1.3 frustum
// clamp, 3 sigma); zenn section 2.3.3 (discriminant floor 0.1).
constexpr int kTile = 16;
constexpr float kDilation = 0.3f;
constexpr float kZNear = 0.05f;
constexpr float kFrustumClamp = 1.3f;
constexpr float kDiscFloor = 0.1f;
constexpr float kSigma = 3.0f;
constexpr float kAlphaMin = 1.0f / 255.0f;
constexpr float kAlphaMax = 0.99f;
constexpr float kTStop = 1e-4f;
// Entries per chunk of a tile's list: the forward keeps each pixel's state
// at these boundaries and the chunked backward walks one chunk per workgroup.
constexpr int kChunk = 256;
// Chunk index of a work item that is a whole list.
constexpr uint32_t kWholeList = 0xffffffffu;

inline int tiles_x(const gs_camera& c) { return (c.width + kTile - 1) / kTile; }
inline int tiles_y(const gs_camera& c) { return (c.height + kTile - 1) / kTile; }

// Tile span [x0, x1) x [y0, y1) covered by the 2r square around (u, v):
// lo = clamp(floor((u - r) / 16), 0, TX), hi = clamp(floor((u + r) / 16) + 1,
// 0, TX), clamped in float then converted (learn-gs tile_spans). Used by the
// preprocess (to count) and by the duplication (to enumerate), so both see
// the same span.
struct Span {
    int x0, x1, y0, y1;
};

__device__ __forceinline__ Span tile_span(float u, float v, float r, int TX, int TY) {
    const float tile = (float)kTile;
    float x0 = floorf((u - r) / tile);
    float x1 = floorf((u + r) / tile) + 1.0f;
    float y0 = floorf((v - r) / tile);
    float y1 = floorf((v + r) / tile) + 1.0f;
    x0 = fminf(fmaxf(x0, 0.0f), (float)TX);
    x1 = fminf(fmaxf(x1, 0.0f), (float)TX);
    y0 = fminf(fmaxf(y0, 0.0f), (float)TY);
    y1 = fminf(fmaxf(y1, 0.0f), (float)TY);
    return Span{(int)x0, (int)x1, (int)y0, (int)y1};
}

// Ellipse tile test (zenn 2.3.4: of the span's tiles keep those the splat's
// ellipse may overlap). The ellipse taken is the region where the splat can
// reach alpha >= 1/255: Q(d) = A dx^2 + 2B dx dy + C dy^2 <= 2 ln(255 o), with
// the opacity-independent bound 2 ln 255 = 11.0825 < 11.1, raised by 64 ulp
// of |A| dx^2 + |C| dy^2 + 2|B dx dy| at the span's farthest pixel centre (the
// compositing's rounding of Q). A dropped tile therefore holds no pixel the
// splat changes: results are those of the full span; only the lists shrink.
// Per row of tiles the kept tiles are a run: those whose pixel centres meet
// the x-extent [L, R] of the ellipse's slice over the row's pixel-centre
// y-range, L and R taken at the dy of the leftmost / rightmost point clamped
// into the row, widened by a slack. Float32, + - * / sqrt (correctly rounded)
// floor ceil fminf fmaxf only, in a fixed order: preprocess (counting) and
// duplication (enumerating) take the identical decision, and so does any
// host evaluation of the same steps. A conic that is not positive definite,
// or a non-finite extent, keeps the whole span.
struct EllipseRows {
    bool full;
    float u, v, A, B, C, det, hx, hy, ydr, slack, thr;
};

__device__ __forceinline__ EllipseRows ellipse_rows(float u, float v, float A, float B, float C, const Span& sp) {
    EllipseRows e;
    e.u = u; e.v = v; e.A = A; e.B = B; e.C = C;
    e.det = A * C - B * B;
    e.full = !(e.det > 0.0f && A > 0.0f && C > 0.0f);
    const float ex = fmaxf(fabsf(16.0f * (float)sp.x0 - u), fabsf(16.0f * (float)sp.x1 - 1.0f - u));
    const float ey = fmaxf(fabsf(16.0f * (float)sp.y0 - v), fabsf(16.0f * (float)sp.y1 - 1.0f - v));
    const float bound = 64.0f * 5.96e-8f * ((fabsf(A) + fabsf(C)) + 2.0f * fabsf(B)) * (ex * ex + ey * ey);
    e.thr = 11.1f + bound;
    e.hx = e.hy = e.ydr = e.slack = 0.0f;
    if (e.full) return e;
    e.hy = sqrtf((e.thr * A) / e.det);
    e.hx = sqrtf((e.thr * C) / e.det);
    e.ydr = -(B * e.hx) / C;
    e.slack = 0.01f + 1e-4f * (e.hx + e.hy);
    if (!isfinite(e.hx) || !isfinite(e.hy) || !isfinite(e.ydr) || !isfinite(e.slack)) e.full = true;
    return e;
}

// Kept tiles [lo, hi) of row ty; hi <= lo means none.
__device__ __forceinline__ void ellipse_row_range(const EllipseRows& e, const Span& sp, int ty, int& lo_out,
                                                  int& hi_out) {
    lo_out = sp.x0;
    hi_out = sp.x0;
    if (e.full) { hi_out = sp.x1; return; }
    const float ylo = 16.0f * (float)ty - e.v;
    const float lo = fmaxf(ylo, -e.hy), hi = fminf(ylo + 15.0f, e.hy);
    if (lo > hi + e.slack) return;
    const float yr = fminf(fmaxf(e.ydr, lo), hi);
    const float yl = fminf(fmaxf(-e.ydr, lo), hi);
    const float thrA = e.thr * e.A;
    const float R = (-(e.B * yr) + sqrtf(fmaxf(0.0f, thrA - (e.det * yr) * yr))) / e.A + e.slack;
    const float L = (-(e.B * yl) - sqrtf(fmaxf(0.0f, thrA - (e.det * yl) * yl))) / e.A - e.slack;
    const float tlo = fmaxf(ceilf(((L + e.u) - 15.0f) / 16.0f), (float)sp.x0);
    const float thi = fminf(floorf((R + e.u) / 16.0f) + 1.0f, (float)sp.x1);
    if (!(tlo < thi)) return;
    lo_out = (int)tlo;
    hi_out = (int)thi;
}

// Tile-test modes (the flags argument of the _ex entry points).
constexpr uint32_t kTilesEllipse = 1u;

// ---- launchers (each returns the launch's hipError_t) ----

// A stack of cameras passed by value to a kernel (at most GS_MAX_VIEWS).
struct CameraSet {
    gs_camera cam[GS_MAX_VIEWS];
    int n;
};
// Records of n Gaussians for every camera of the set, camera v's at v n + g.
hipError_t launch_preprocess_views(const CameraSet& cams, int n, const float* means, const float* scales,
                                   const float* quats, const float* opacity, const float* sh, int sh_degree,
                                   const float* rgb_in, float4* xy_depth, float4* conic_op, float4* rgb,
                                   uint32_t* tiles_touched, uint32_t flags, hipStream_t stream);
hipError_t launch_preprocess(const gs_camera& cam, int n, const float* means, const float* scales,
                             const float* quats, const float* opacity, const float* sh,
                             int sh_degree, const float* rgb_in, float4* xy_depth,
                             float4* conic_op, float4* rgb, uint32_t* tiles_touched,
                             uint32_t flags, hipStream_t stream);

hipError_t launch_preprocess_bwd(const gs_camera& cam, int n, const float* means, const float* scales,
                                 const float* quats, const float* sh, int sh_degree,
                                 const uint32_t* tiles_touched, const float2* grad_mean2d,
                                 const float4* grad_conic_op, const float4* grad_rgb, float* grad_means,
                                 float* grad_scales, float* grad_quats, float* grad_opacity,
                                 float* grad_sh, float* grad_rgb_in, hipStream_t stream);

// Binning workspace, carved from the caller's scratch buffer. Nothing in it
// needs initialisation: every word is written before it is read within one
// call.
struct BinScratch {
    uint64_t* total;          // [1] entry count
    uint32_t* gauss_hist;     // [4][256] digit totals of the depth passes
    uint32_t* entry_hist;     // [3][256] digit totals of the tile-id passes
    uint32_t* gauss_counts;   // [4][256][nb_gauss] per-tile digit counts, then prefixes
    uint32_t* entry_counts;   // [3][256][nb_entry]
    uint32_t* tt_counts;      // [256][nb_gauss] per-tile sums of tiles_touched, last depth pass
    uint64_t* tt_prefix;      // [256][nb_gauss] their exclusive prefix over tiles
    uint64_t* tt_hist;        // [256] their totals
    uint32_t* offsets;        // [n] first entry of the i-th splat in depth order
    uint32_t* first_owner;    // [nb_entry] owner (depth-order index) of each 2048-entry tile's first entry
    uint32_t* gk[2];          // [n] depth keys, ping-pong
    uint32_t* gv[2];          // [n] splat ids, ping-pong; gv[0] ends as the depth order
    uint64_t* keys_tmp;       // [capacity]
    uint32_t* vals_tmp;       // [capacity]
};
size_t bin_scratch_layout(int n, int64_t capacity, BinScratch* out, void* base);

// The whole binning: stable depth order of the splats with the scan of
// their tile counts in that order (E -> *s.total, and *n_dev if given), duplication,
// stable sort on the tile-id bits into (keys, values). Never waits on the
// host. When E > capacity nothing is written to keys/values. The n splats
// may be a stack of n_views views of cam's size (n / n_views each, view v's
// tiles in the band of rows [v TY, v TY + TY)).
hipError_t launch_bin_and_sort(const gs_camera& cam, int n_views, int n, const float4* xy_depth,
                               const float4* conic_op, const uint32_t* tiles_touched, uint64_t* keys,
                               uint32_t* values, uint32_t capacity, const BinScratch& s, uint64_t* n_dev,
                               uint32_t flags, hipStream_t stream);

hipError_t launch_fill_u32(uint32_t* p, size_t words, uint32_t v, hipStream_t stream);

// Per-tile ranges. The entry count is n_entries, or, when n_dev is given,
// *n_dev if it does not exceed capacity and 0 otherwise. If tile_order is
// given it receives the tiles, heaviest list first; if chunks is given, the
// count and (tile, chunk) pairs of every kChunk-entry chunk of every list.
hipError_t launch_tile_ranges(const uint64_t* keys, uint32_t n_entries, const uint64_t* n_dev, uint32_t capacity,
                              int n_tiles, uint32_t* ranges, uint32_t* tile_order, uint32_t* chunks,
                              hipStream_t stream);

// Compositing over a stack of n_views views of cam's size (each a band of
// tiles_y(cam) tile rows; per-view planes one after another). With ckpt,
// the forward also stores the per-pixel state at
// every kChunk-entry boundary of a list and the backward runs one workgroup
// per chunk of the schedule `chunks` (capacity: length of the sorted entry
// arrays).
hipError_t launch_composite_fwd(const gs_camera& cam, int n_views, const uint32_t* ranges,
                                const uint32_t* point_list, const float4* xy_depth,
                                const float4* conic_op, const float4* rgb, float3 bg,
                                float* image, float* final_T, uint32_t* n_contrib,
                                uint32_t* n_examined, const uint32_t* tile_order, float4* ckpt,
                                uint32_t capacity, const uint32_t* chunks, void* part, hipStream_t stream);
// Bytes of the chunk partials the scheduled forward needs.
size_t composite_part_bytes(const gs_camera& cam, int n_views, uint32_t capacity);

hipError_t launch_composite_bwd(const gs_camera& cam, int n_views, int n, const uint32_t* ranges,
                                const uint32_t* point_list, const float4* xy_depth,
                                const float4* conic_op, const float4* rgb, float3 bg,
                                const float* final_T, const uint32_t* n_contrib,
                                const float* dL_dimage, float2* grad_mean2d,
                                float4* grad_conic_op, float4* grad_rgb, const uint32_t* tile_order,
                                const uint32_t* chunks, uint32_t capacity, const float4* ckpt,
                                const float* image, hipStream_t stream);

// Appearance MLP: parameter count, backward scratch (per-workgroup partial
// weight gradients) and launchers.
int appearance_params(int L, int H);
size_t appearance_bwd_scratch(int n, int L, int H);
hipError_t launch_appearance_fwd(const gs_camera& cam, int n, const float* means, const float* latent, int L,
                                 int H, const float* weights, float* rgb, hipStream_t stream);
hipError_t launch_appearance_bwd(const gs_camera& cam, int n, const float* means, const float* latent, int L,
                                 int H, const float* weights, const float* grad_rgb, float* grad_latent,
                                 float* grad_weights, float* partials, hipStream_t stream);

}  // namespace gs
