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

// Workgroups are handed to the 8 XCDs round-robin by workgroup id. Remap
// the id so each XCD walks one contiguous run of tiles: neighbouring tiles
// share most of their splats, and each XCD has its own L2.
__device__ __forceinline__ int xcd_contiguous(int bid, int nblocks) {
    const int q = nblocks / 8, rem = nblocks % 8;
    const int x = bid % 8, i = bid / 8;
    return x * q + (x < rem ? x : rem) + i;
}

// ---- launchers (each returns the launch's hipError_t) ----

hipError_t launch_preprocess(const gs_camera& cam, int n, const float* means, const float* scales,
                             const float* quats, const float* opacity, const float* sh,
                             int sh_degree, const float* rgb_in, float4* xy_depth,
                             float4* conic_op, float4* rgb, uint32_t* tiles_touched,
                             hipStream_t stream);

// Binning workspace, carved from the caller's scratch buffer.
struct BinScratch {
    uint32_t* block_sums;     // [nb_scan]
    uint64_t* block_offsets;  // [nb_scan]
    uint64_t* total;          // [1]
    uint32_t* offsets;        // [n] first entry of each Gaussian
    uint64_t* keys_tmp;       // [capacity]
    uint32_t* vals_tmp;       // [capacity]
    uint32_t* counts;         // [256][nb_sort]
    uint32_t* digit_totals;   // [256]
    uint32_t* seg_ranges;     // [n_tiles][2] tile segments after the tile-id passes
    uint32_t* seg_k0;         // [capacity] global ping-pong of the per-tile sort
    uint32_t* seg_v0;
    uint32_t* seg_k1;
    uint32_t* seg_v1;
};
size_t bin_scratch_layout(int n, int64_t capacity, int n_tiles, BinScratch* out, void* base);

// Exclusive scan of tiles_touched into s.offsets and s.total (entry count).
hipError_t launch_scan(int n, const uint32_t* tiles_touched, const BinScratch& s, hipStream_t stream);
// One (key, value) per entry, n_entries = *s.total, written to keys/values.
hipError_t launch_duplicate(const gs_camera& cam, int n, uint32_t n_entries, const float4* xy_depth,
                            const BinScratch& s, uint64_t* keys, uint32_t* values, hipStream_t stream);

// Sort n entries by the whole key (tile id << 32 | depth bits), stably.
// The duplication must have written the entries into the tmp pair when
// dup_writes_tmp(tile_bits), into (keys, values) otherwise; the result is in
// (keys, values).
int tile_pass_count(int tile_bits);
bool dup_writes_tmp(int tile_bits);
hipError_t launch_sort(uint64_t* keys, uint32_t* values, uint32_t n, int tile_bits, int n_tiles,
                       const BinScratch& s, hipStream_t stream);

hipError_t launch_tile_ranges(const uint64_t* keys, uint32_t n_entries, int n_tiles,
                              uint32_t* ranges, hipStream_t stream);

hipError_t launch_composite_fwd(const gs_camera& cam, const uint32_t* ranges,
                                const uint32_t* point_list, const float4* xy_depth,
                                const float4* conic_op, const float4* rgb, float3 bg,
                                float* image, float* final_T, uint32_t* n_contrib,
                                uint32_t* n_examined, hipStream_t stream);

hipError_t launch_composite_bwd(const gs_camera& cam, int n, const uint32_t* ranges,
                                const uint32_t* point_list, const float4* xy_depth,
                                const float4* conic_op, const float4* rgb, float3 bg,
                                const float* final_T, const uint32_t* n_contrib,
                                const float* dL_dimage, float2* grad_mean2d,
                                float4* grad_conic_op, float4* grad_rgb, hipStream_t stream);

}  // namespace gs
