/*
 * gs.h - C ABI of libgs, a tile-based 3D Gaussian Splatting rasterizer for
 * AMD Instinct MI355X (gfx950), forward and backward.
 *
 * The pipeline follows the pages it was built from:
 *   - "rigel" (GitHub README), sections "Projection", "Binning",
 *     "Rasterization", "Backward" and "Deliberate differences";
 *   - "3D Gaussian Splatting ビューワを作る" (zenn.dev), sections 2.1-2.3
 *     (preprocess), 4.1 (prefix scan), 4.2 (duplicate), 4.3 (radix sort),
 *     4.4 (tile ranges) and 4.5 (tile render);
 *   - "11 - Tiles: the actual 3DGS design" (learn-gs notebook): constants,
 *     prep_splats, tile_spans, build_tile_lists and the tiled kernel loop.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Memory: every array argument is a DEVICE pointer unless marked (host).
 *    The caller owns all memory; libgs never allocates device memory.
 *    Scratch space follows a size-query protocol: call with scratch == NULL
 *    to receive the required byte count in *scratch_bytes; nothing is
 *    launched by such a call.
 *  - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream). Work is enqueued asynchronously; the only call that blocks the
 *    host is gs_bin_and_sort, which waits once to read the entry count.
 *    gs_bin_and_sort_async and gs_tile_ranges_async keep that count in
 *    device memory instead, so a whole frame is enqueued without a wait.
 *  - Errors: every call returns a gs_status. Arguments are validated on the
 *    host before anything is launched; on GS_ERR_INVALID nothing was
 *    enqueued. gs_last_error() gives a message for the calling thread. HIP
 *    failures are reported as GS_ERR_HIP.
 *  - Layouts: per-Gaussian inputs are structure-of-arrays, component-major
 *    float32: means/scales [3][n], quats [4][n] as (w, x, y, z), opacity
 *    [n], sh [(d+1)^2][3][n]. Per-Gaussian outputs are packed float4
 *    records [n][4]. Images are planar [3][H][W] float32; per-pixel buffers
 *    are [H][W]. Every output is overwritten, never accumulated into.
 *  - Tiles are 16 x 16 pixels; TX = ceil(W / 16), TY = ceil(H / 16); tile id
 *    t = ty * TX + tx. Pixel (x, y) is sampled at the integer point (x, y).
 *  - Limits: 0 <= n <= GS_MAX_GAUSSIANS; 1 <= width, height <= GS_MAX_DIM.
 */
#ifndef GS_H
#define GS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GS_TILE 16
#define GS_MAX_GAUSSIANS (1 << 24) /* prefix-scan capacity, 256^3 */
#define GS_MAX_DIM 16384
#define GS_MAX_VIEWS 32 /* cameras of one view stack */

/* Tile tests (the flags of the _ex entry points). GS_TILES_SQUARE: a splat
 * is listed in every tile of its span rectangle. GS_TILES_ELLIPSE: only in
 * the tiles of the span that the region where it can reach alpha >= 1/255
 * overlaps (zenn 2.3.4, "keep only tiles the ellipse may intersect"); the
 * ellipse is Q(d) <= 11.1 + r, with Q(d) = d^T conic d, 11.1 > 2 ln 255 an
 * opacity-independent bound and r a bound on the compositing's float32
 * rounding of Q. A dropped tile holds no pixel the splat changes, so image,
 * final_T and every gradient equal those of GS_TILES_SQUARE; the lists are
 * shorter (E drops by about 40% on the 160k-Gaussian 1080p scene) and
 * n_contrib, being a list position, changes with them. Per row of the span
 * the kept tiles are a run: those whose pixel centres meet the x-extent of
 * the ellipse's slice over the row's pixel-centre y-range (the slice's
 * edges taken at the ellipse's leftmost / rightmost points clamped into the
 * row, widened by 0.01 + 1e-4 (hx + hy) pixels), evaluated in float32 with
 * correctly rounded division and square root in a fixed order. */
#define GS_TILES_SQUARE 0u
#define GS_TILES_ELLIPSE 1u

/* Appearance MLP limits ("rigel" README, "Appearance MLP": sized for up to
 * 29 latent dims and 64 hidden units). */
#define GS_APP_MAX_LATENT 29
#define GS_APP_MAX_HIDDEN 64

typedef enum {
    GS_OK = 0,
    GS_ERR_INVALID = 1,  /* bad argument; nothing enqueued */
    GS_ERR_CAPACITY = 2, /* entry count exceeds the caller's capacity */
    GS_ERR_OVERFLOW = 3, /* entry count does not fit in 32 bits */
    GS_ERR_HIP = 4       /* a HIP runtime call failed */
} gs_status;

/* Pinhole camera, passed by host pointer. p_cam = R p + t with R row-major
 * world-to-camera; +z looks forward, image y grows downward. campos is the
 * camera centre in world space (-R^T t), used for the SH view direction.
 * fx, fy, cx, cy are in pixels and must be finite with fx, fy > 0.
 * ("rigel" README, "Deliberate differences": row-major world-to-camera
 * matrices and explicit pinhole intrinsics.) */
typedef struct {
    float R[9];
    float t[3];
    float campos[3];
    float fx, fy, cx, cy;
    int32_t width, height;
} gs_camera;

/* Library constants, in this order: tile size, dilation (0.3), near plane
 * (0.05), frustum clamp (1.3), discriminant floor (0.1), sigma (3), alpha
 * floor (1/255), alpha cap (0.99), transmittance stop (1e-4). (learn-gs
 * constants block; "rigel" README "Projection"; zenn section 2.3.3.)
 * out: host array of 9 floats. */
void gs_constants(float out[9]);

/* Message describing the last failure on the calling thread ("" if none). */
const char* gs_last_error(void);

/* Library version as (major, minor, patch), written to out (host). */
void gs_version(int32_t out[3]);

/* ---------------------------------------------------------------------
 * gs_preprocess - project every Gaussian to a screen-space splat.
 * ("rigel" README "Projection"; zenn 2.1.1-2.1.2, 2.2.3, 2.3.1, 2.3.3;
 * learn-gs prep_splats and tile_spans.)
 *
 * Per Gaussian g: camera transform; cull unless z > 0.05; pinhole centre
 * (u, v); quaternion normalised to R(q); Sigma = R S S^T R^T; J built at the
 * centre with x/z and y/z clamped to 1.3x the frustum half-width;
 * Sigma_2d = (J W) Sigma (J W)^T + 0.3 I; cull unless det > 0; conic
 * (A, B, C) = (c, -b, a) / det; radius r = ceil(3 sqrt(lambda_max)) with the
 * discriminant floored at 0.1; tile span [x0, x1) x [y0, y1) with
 * x0 = clamp(floor((u - r) / 16), 0, TX), x1 = clamp(floor((u + r) / 16) + 1,
 * 0, TX) (same in y); cull if the span is empty. Colour from SH degree
 * 0..sh_degree at the unit direction (mean - campos), or copied from rgb_in.
 * Any non-finite intermediate or output also culls. A culled Gaussian's
 * outputs are all zero.
 *
 *   cam            (host) camera
 *   n              number of Gaussians
 *   means, scales  [3][n] float32; scales are positive (already activated)
 *   quats          [4][n] float32 (w, x, y, z), need not be unit
 *   opacity        [n] float32 in (0, 1) (already activated)
 *   sh             [(sh_degree+1)^2][3][n] float32, or NULL
 *   sh_degree      0..3 (ignored when sh == NULL)
 *   rgb_in         [3][n] float32; required iff sh == NULL
 *   xy_depth       out [n][4]: (u, v, z, r)
 *   conic_op       out [n][4]: (A, B, C, opacity)
 *   rgb            out [n][4]: (r, g, b, 0)
 *   tiles_touched  out [n] uint32: span area (0 = culled)
 * Every floating-point result is computed in float32 with a fixed operation
 * order and no contraction, so it is bit-identical to a host evaluation of
 * the same formulas.
 * ------------------------------------------------------------------- */
gs_status gs_preprocess(const gs_camera* cam, int32_t n, const float* means, const float* scales,
                        const float* quats, const float* opacity, const float* sh,
                        int32_t sh_degree, const float* rgb_in, float* xy_depth, float* conic_op,
                        float* rgb, uint32_t* tiles_touched, void* stream);

/* gs_preprocess_ex - gs_preprocess with a tile test (flags: GS_TILES_SQUARE
 * or GS_TILES_ELLIPSE). With GS_TILES_ELLIPSE, tiles_touched counts the
 * kept tiles only, and a Gaussian with none kept is culled (all outputs
 * zero). Any other flag bit is GS_ERR_INVALID. */
gs_status gs_preprocess_ex(const gs_camera* cam, int32_t n, const float* means, const float* scales,
                           const float* quats, const float* opacity, const float* sh,
                           int32_t sh_degree, const float* rgb_in, float* xy_depth, float* conic_op,
                           float* rgb, uint32_t* tiles_touched, uint32_t flags, void* stream);

/* ---------------------------------------------------------------------
 * gs_preprocess_views - gs_preprocess_ex for a stack of n_views cameras of
 * one size at once: each Gaussian's inputs are read once and its record for
 * camera v is written at index v n + g of every output (xy_depth, conic_op,
 * rgb [n_views n][4], tiles_touched [n_views n]), the same bits
 * gs_preprocess_ex writes for that camera alone. Such a stack is binned,
 * ranged and composited as one frame whose view v owns the band of tile
 * rows [v TY, v TY + TY) (gs_bin_and_sort_views_async, gs_tile_ranges_ex,
 * gs_composite_fwd_ex, gs_composite_bwd_ex with n_views).
 *
 *   cams       (host) n_views cameras, 1 <= n_views <= GS_MAX_VIEWS, all of
 *              the same width and height
 *   n          Gaussians; n_views n <= GS_MAX_GAUSSIANS
 * Other arguments as gs_preprocess_ex.
 * ------------------------------------------------------------------- */
gs_status gs_preprocess_views(const gs_camera* cams, int32_t n_views, int32_t n, const float* means,
                              const float* scales, const float* quats, const float* opacity, const float* sh,
                              int32_t sh_degree, const float* rgb_in, float* xy_depth, float* conic_op, float* rgb,
                              uint32_t* tiles_touched, uint32_t flags, void* stream);

/* ---------------------------------------------------------------------
 * gs_preprocess_bwd - gradients of gs_preprocess's outputs with respect to
 * the Gaussians' parameters (the projection backward).
 * ("rigel" README "Backward", its last paragraph, and "Deliberate
 * differences" (quaternion normalisation in the backward); zenn 2.2.3 for
 * the SH basis.)
 *
 * Chains dL/d(u, v), dL/d(A, B, C) and dL/d(colour) through the 2x2
 * inverse, Sigma_2d = T Sigma T^T with T = J W, the Jacobian's dependence on
 * the camera-space centre (when x/z or y/z was clamped, that entry of J sends
 * its gradient to z only), the pinhole, the camera transform, and
 * Sigma = M M^T, M = R(q) S, down to the scales and the raw quaternion
 * (through its normalisation). The colour gradient reaches the SH
 * coefficients and, through the view direction normalize(mean - campos),
 * the mean. dL/dopacity is passed through from grad_conic_op. A Gaussian
 * with tiles_touched == 0 (culled by the forward) gets zero gradients.
 * Computed in float32; each Gaussian's gradients are formed by one thread
 * (no atomics, deterministic).
 *
 *   cam, n, means, scales, quats, sh, sh_degree: as given to gs_preprocess
 *   tiles_touched   [n] from gs_preprocess
 *   grad_mean2d     [n][2] dL/d(u, v) (from gs_composite_bwd)
 *   grad_conic_op   [n][4] dL/d(A, B, C, opacity)
 *   grad_rgb        [n][4] dL/d(r, g, b, -)
 *   grad_means      out [3][n]
 *   grad_scales     out [3][n]
 *   grad_quats      out [4][n] (w, x, y, z); orthogonal to the quaternion
 *   grad_opacity    out [n]
 *   grad_sh         out [(sh_degree+1)^2][3][n]; required iff sh != NULL
 *   grad_rgb_in     out [3][n]; required iff sh == NULL (dL/d rgb_in)
 * Every output is overwritten.
 * ------------------------------------------------------------------- */
gs_status gs_preprocess_bwd(const gs_camera* cam, int32_t n, const float* means, const float* scales,
                            const float* quats, const float* sh, int32_t sh_degree,
                            const uint32_t* tiles_touched, const float* grad_mean2d,
                            const float* grad_conic_op, const float* grad_rgb, float* grad_means,
                            float* grad_scales, float* grad_quats, float* grad_opacity, float* grad_sh,
                            float* grad_rgb_in, void* stream);

/* ---------------------------------------------------------------------
 * gs_bin_and_sort - duplicate splats into tile entries and sort them.
 * ("rigel" README "Binning"; zenn 4.1-4.3; learn-gs build_tile_lists.)
 *
 * Exclusive prefix sum of tiles_touched gives Gaussian g the private slice
 * [offset_g, offset_g + tiles_touched[g]) of the entry array; g writes one
 * entry per tile of its span, ty outer and tx inner, with
 *     key   = (uint64)(ty * TX + tx) << 32 | float_bits(z_g)
 *     value = g.
 * The result is the entries in the order of one stable sort by key, so
 * equal keys keep Gaussian-index order: (tile, depth bits, g). It is
 * reached by a stable radix sort of the Gaussians by depth bits, emission
 * in that order, and a stable radix sort of the entries on the
 * ceil(log2(TX*TY)) tile-id bits. Everything is enqueued first; then the
 * entry count E is copied to the host: this is the call's one host
 * synchronisation.
 *
 *   cam, n         as gs_preprocess; n <= GS_MAX_GAUSSIANS
 *   xy_depth       [n][4] from gs_preprocess
 *   tiles_touched  [n] from gs_preprocess
 *   keys           out [capacity] uint64: sorted keys (first E valid)
 *   point_list     out [capacity] uint32: Gaussian ids in sorted order
 *   capacity       entries the caller allocated
 *   scratch        device workspace of *scratch_bytes bytes (256-byte
 *                  aligned), or NULL to query the size
 *   scratch_bytes  (host) in: size of scratch; out: required size, which
 *                  depends on n and capacity
 *   n_entries      (host) out: E
 * Returns GS_ERR_CAPACITY (with *n_entries = E; keys/point_list are then
 * not written) when E > capacity and GS_ERR_OVERFLOW when E >= 2^32.
 * Calls that share one scratch buffer must not overlap.
 * ------------------------------------------------------------------- */
gs_status gs_bin_and_sort(const gs_camera* cam, int32_t n, const float* xy_depth,
                          const uint32_t* tiles_touched, uint64_t* keys, uint32_t* point_list,
                          int64_t capacity, void* scratch, size_t* scratch_bytes,
                          int64_t* n_entries, void* stream);

/* gs_bin_and_sort_ex - gs_bin_and_sort with a tile test; must match the
 * flags given to gs_preprocess_ex for the same splats. With
 * GS_TILES_ELLIPSE each Gaussian writes its kept tiles only (rows ty outer,
 * tx inner), which needs conic_op ([n][4] from gs_preprocess_ex, 16-byte
 * aligned); conic_op may be NULL with GS_TILES_SQUARE. */
gs_status gs_bin_and_sort_ex(const gs_camera* cam, int32_t n, const float* xy_depth, const float* conic_op,
                             const uint32_t* tiles_touched, uint64_t* keys, uint32_t* point_list,
                             int64_t capacity, void* scratch, size_t* scratch_bytes, int64_t* n_entries,
                             uint32_t flags, void* stream);

/* ---------------------------------------------------------------------
 * gs_bin_and_sort_async - gs_bin_and_sort without the host wait.
 *
 * Same work, order and arguments as gs_bin_and_sort, except that E is
 * written to device memory and the host never waits:
 *   n_entries_dev  out, device uint64 (8-byte aligned): E, written on the
 *                  stream.
 * When E > capacity keys and point_list are not written;
 * gs_tile_ranges_async then marks every tile empty, so the frame renders the
 * background and the caller, once it reads E, grows the buffers and renders
 * the frame again. Host-side argument errors are returned as usual; calls
 * that share one scratch buffer must not overlap.
 * ------------------------------------------------------------------- */
gs_status gs_bin_and_sort_async(const gs_camera* cam, int32_t n, const float* xy_depth,
                                const uint32_t* tiles_touched, uint64_t* keys, uint32_t* point_list,
                                int64_t capacity, void* scratch, size_t* scratch_bytes,
                                uint64_t* n_entries_dev, void* stream);

/* gs_bin_and_sort_async_ex - gs_bin_and_sort_async with a tile test, as
 * gs_bin_and_sort_ex. */
gs_status gs_bin_and_sort_async_ex(const gs_camera* cam, int32_t n, const float* xy_depth, const float* conic_op,
                                   const uint32_t* tiles_touched, uint64_t* keys, uint32_t* point_list,
                                   int64_t capacity, void* scratch, size_t* scratch_bytes,
                                   uint64_t* n_entries_dev, uint32_t flags, void* stream);

/* ---------------------------------------------------------------------
 * gs_bin_and_sort_async_noalloc - gs_bin_and_sort_async_ex for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same work, order,
 * results and flags, with the binning workspace taken from a fixed array
 * inside the library instead of a caller-owned scratch buffer.
 *
 * The array holds GS_NOALLOC_SCRATCH_BYTES (128 MiB) on every GPU the
 * library is loaded on, for the life of the process; its address on the
 * current device is looked up on the first call made with that device
 * current. A call whose workspace (the scratch size gs_bin_and_sort_async
 * reports for the same n and capacity) exceeds it returns GS_ERR_INVALID,
 * with a message, before anything is enqueued: about n = 1M Gaussians with
 * capacity = 5M entries fits. The call allocates nothing (no hipMalloc, no
 * hipFree) and needs no cleared memory: every word of the workspace that a
 * kernel reads was written earlier in the same call.
 *
 * All calls on one GPU share that GPU's array, which keeps the last call's
 * contents: two such calls that overlap on one GPU (on different streams,
 * or from different threads without ordering) race and corrupt each other's
 * results. Order them on one stream, or use gs_bin_and_sort_async_ex.
 *
 *   cam, n, xy_depth, conic_op, tiles_touched, keys, point_list, capacity,
 *   n_entries_dev, flags, stream: as gs_bin_and_sort_async_ex
 * ------------------------------------------------------------------- */
#define GS_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
gs_status gs_bin_and_sort_async_noalloc(const gs_camera* cam, int32_t n, const float* xy_depth,
                                        const float* conic_op, const uint32_t* tiles_touched, uint64_t* keys,
                                        uint32_t* point_list, int64_t capacity, uint64_t* n_entries_dev,
                                        uint32_t flags, void* stream);

/* gs_bin_and_sort_views_async - gs_bin_and_sort_async_ex over a stack of
 * n_views views (see gs_preprocess_views): xy_depth, conic_op and
 * tiles_touched hold n_views n records, view v's at v n + g; an entry's
 * tile id is v TX TY + ty TX + tx for the tile (tx, ty) of its own view,
 * and its value the record index v n + g. Within each view's band the
 * lists are exactly those of gs_bin_and_sort_async_ex for that view alone.
 * cam gives the size of one view; TX TY n_views <= 2^24. The scratch size
 * is that of gs_bin_and_sort(_async) for n_views n Gaussians. */
gs_status gs_bin_and_sort_views_async(const gs_camera* cam, int32_t n_views, int32_t n, const float* xy_depth,
                                      const float* conic_op, const uint32_t* tiles_touched, uint64_t* keys,
                                      uint32_t* point_list, int64_t capacity, void* scratch, size_t* scratch_bytes,
                                      uint64_t* n_entries_dev, uint32_t flags, void* stream);

/* ---------------------------------------------------------------------
 * gs_tile_ranges - per-tile [start, end) of the sorted entries.
 * (zenn 4.4.1-4.4.2; "rigel" README "Binning": the range kernel.)
 *
 *   keys        [n_entries] sorted keys from gs_bin_and_sort
 *   n_entries   E
 *   ranges      out [TX*TY][2] uint32: (start, end); (0, 0) for an empty tile
 *   tile_order  out [TX*TY] uint32, or NULL: a schedule for the compositing
 *               calls, every tile once, in descending order of list length
 *               (by classes of 1/16 octave; order within a class
 *               unspecified). It changes no result, only the order in which
 *               tiles are processed: a compositing launch lasts at least as
 *               long as its heaviest tile, so that tile is started first.
 * ------------------------------------------------------------------- */
gs_status gs_tile_ranges(const gs_camera* cam, const uint64_t* keys, int64_t n_entries,
                         uint32_t* ranges, uint32_t* tile_order, void* stream);

/* ---------------------------------------------------------------------
 * gs_tile_ranges_async - gs_tile_ranges with the entry count in device
 * memory, as written by gs_bin_and_sort_async.
 *
 *   keys           [capacity] sorted keys
 *   n_entries_dev  device uint64 (8-byte aligned): E
 *   capacity       the capacity given to gs_bin_and_sort_async
 *   ranges         out [TX*TY][2] uint32; every tile (0, 0) when E > capacity
 *   tile_order     out [TX*TY] uint32, or NULL: as gs_tile_ranges
 * ------------------------------------------------------------------- */
gs_status gs_tile_ranges_async(const gs_camera* cam, const uint64_t* keys, const uint64_t* n_entries_dev,
                               int64_t capacity, uint32_t* ranges, uint32_t* tile_order, void* stream);

/* ---------------------------------------------------------------------
 * gs_tile_ranges_ex - gs_tile_ranges (n_entries_dev NULL: E = n_entries)
 * or gs_tile_ranges_async (E = *n_entries_dev, every tile empty when it
 * exceeds capacity), optionally with the chunk schedule of the chunked
 * backward (gs_composite_bwd_ex).
 *
 *   n_views     1, or the views of a stack (gs_bin_and_sort_views_async):
 *               the tiles are then the TX TY n_views of the stack
 *   keys, ranges, tile_order  as gs_tile_ranges / gs_tile_ranges_async
 *   capacity    length of keys; n_entries <= capacity when n_entries_dev is
 *               NULL
 *   chunks      out uint32 [4 + 4 * (TX * TY * n_views + ceil(capacity / 256))],
 *               16-byte aligned, or NULL: the work items of
 *               gs_composite_fwd_ex and gs_composite_bwd_ex (the compositing
 *               launches read up to that many items, one per workgroup).
 *               chunks[0] = the item count; words 1-3 unused; from word 4,
 *               for each item, (tile, k, list start, L). When the lists
 *               average more than 256 entries (E > 256 TX TY n_views),
 *               every list longer than 256 is cut into ceil(L / 256)
 *               chunks, chunk k covering list positions [256 k,
 *               min(256 k + 256, L)), and every shorter list (empty ones
 *               too) is one item with k = 0xffffffff (the whole list);
 *               otherwise every list is one such item. Items come in
 *               descending order of L - 256 k, the list length from the item
 *               on (classes as tile_order's; k = 0 for whole lists).
 * ------------------------------------------------------------------- */
gs_status gs_tile_ranges_ex(const gs_camera* cam, int32_t n_views, const uint64_t* keys, int64_t n_entries,
                            const uint64_t* n_entries_dev, int64_t capacity, uint32_t* ranges,
                            uint32_t* tile_order, uint32_t* chunks, void* stream);

/* ---------------------------------------------------------------------
 * gs_composite_fwd - front-to-back alpha compositing per tile.
 * ("rigel" README "Rasterization"; zenn 4.5; learn-gs "The kernel".)
 *
 * For pixel (x, y) in tile t, over j = start_t .. end_t - 1 with
 * g = point_list[j]: dx = x - u_g, dy = y - v_g,
 * power = -0.5 (A dx^2 + C dy^2) - B dx dy, alpha = min(0.99, o exp(power));
 * alpha < 1/255 is skipped; otherwise C += c alpha T, T *= 1 - alpha, and
 * the pixel stops once T < 1e-4 (the splat that crossed is included).
 * image = C + T bg.
 *
 *   ranges, point_list     from gs_tile_ranges / gs_bin_and_sort
 *   xy_depth, conic_op, rgb  [n][4] from gs_preprocess
 *   bg          (host) 3 floats, background colour
 *   image       out [3][H][W]
 *   final_T     out [H][W]: transmittance left at the pixel
 *   n_contrib   out [H][W] uint32: 1 + list position (within the tile) of
 *               the last contributing splat, 0 if none
 *   n_examined  out [H][W] uint32, or NULL: splats evaluated before the
 *               pixel stopped (diagnostic; pixel-splat evaluations)
 *   tile_order  [TX*TY] uint32 from gs_tile_ranges, or NULL (tile-id order):
 *               the order tiles are processed in; any permutation of the
 *               tiles gives the same results
 * ------------------------------------------------------------------- */
gs_status gs_composite_fwd(const gs_camera* cam, const uint32_t* ranges, const uint32_t* point_list,
                           const float* xy_depth, const float* conic_op, const float* rgb,
                           const float bg[3], float* image, float* final_T, uint32_t* n_contrib,
                           uint32_t* n_examined, const uint32_t* tile_order, void* stream);

/* ---------------------------------------------------------------------
 * gs_composite_bwd - reverse walk of the compositing, per tile.
 * ("rigel" README "Backward" and "Deliberate differences"; learn-gs "The
 * next live problem".)
 *
 * Each pixel walks its tile's list from n_contrib - 1 down to 0, undoing
 * T_j = T_{j+1} / (1 - alpha_j) from final_T and carrying the colour behind
 * the current splat (starting from bg). With g_pix = dL/dI:
 *   dL/dc      += alpha T_j g_pix
 *   dL/dalpha   = T_j sum_ch g_pix,ch (c_ch - behind_ch)
 * and, unless the alpha was clamped (o G > 0.99, then nothing more):
 *   dL/do += G dL/dalpha; with dp = alpha dL/dalpha:
 *   dA += -0.5 dx^2 dp, dB += -dx dy dp, dC += -0.5 dy^2 dp,
 *   du += (A dx + B dy) dp, dv += (B dx + C dy) dp.
 * Sums over all pixels are formed on the device; the summation order is
 * not fixed, so results agree with an exact sum to float32 rounding.
 *
 *   n                 number of Gaussians (size of the gradient arrays)
 *   ranges, point_list, xy_depth, conic_op, rgb, bg: as gs_composite_fwd
 *   final_T, n_contrib  from gs_composite_fwd
 *   dL_dimage         [3][H][W] upstream gradient
 *   grad_mean2d       out [n][2]: (du, dv)
 *   grad_conic_op     out [n][4]: (dA, dB, dC, dopacity)
 *   grad_rgb          out [n][4]: (dr, dg, db, 0)
 *   tile_order        as gs_composite_fwd, or NULL
 * ------------------------------------------------------------------- */
gs_status gs_composite_bwd(const gs_camera* cam, int32_t n, const uint32_t* ranges,
                           const uint32_t* point_list, const float* xy_depth,
                           const float* conic_op, const float* rgb, const float bg[3],
                           const float* final_T, const uint32_t* n_contrib,
                           const float* dL_dimage, float* grad_mean2d, float* grad_conic_op,
                           float* grad_rgb, const uint32_t* tile_order, void* stream);

/* ---------------------------------------------------------------------
 * gs_composite_fwd_ex - gs_composite_fwd that can keep, for the chunked
 * backward (gs_composite_bwd_ex), each pixel's state at every 256-entry
 * boundary of its tile's list, and can composite long lists in 256-entry
 * chunks in parallel. The compositing is that of gs_composite_fwd ("rigel"
 * README "Rasterization").
 *
 *   n_views   1, or the views of a stack: cam gives one view's size, the
 *             tiles, ranges and schedule cover the stack, and image
 *             [n_views][3][H][W], final_T, n_contrib, n_examined
 *             [n_views][H][W] hold view after view
 *   capacity  length of the sorted entry arrays (keys, point_list): the
 *             entry count E, or the capacity the asynchronous binning used;
 *             every tile range must lie in [0, capacity)
 *   ckpt      out float32 [ceil(capacity / 256) * 256][4], or NULL. For tile
 *             t and a boundary b = start_t + 256 k (k >= 1, b < end_t) that
 *             the pixel's compositing reached, row (b / 256) * 256 + q holds
 *             (T, C_r, C_g, C_b) of the tile's pixel q in front of entry b, C
 *             the colour accumulated so far; q = 64 w + 8 r + c is pixel
 *             (8 (w & 1) + c, 8 (w >> 1) + r) of the tile. Distinct boundaries
 *             never share a row (those of one list are 256 apart, the next
 *             list's lie more than 256 further on). Other rows are left as
 *             they were.
 *   chunks    the schedule gs_tile_ranges_ex wrote for this frame, or NULL
 *             (tiles in tile_order, each list walked whole). With it every
 *             work item is one workgroup: whole lists as without it; a chunk
 *             is first composited on its own from T = 1 (a pixel stopping
 *             where that local T falls below 1e-4), then each pixel combines
 *             the chunks in front of it (T_in *= T_chunk, C += T_in C_chunk)
 *             and, in the chunk where T_in T_chunk falls below 1e-4, is
 *             composited again splat by splat from (T_in, C) and stops where
 *             the whole-list walk stops. Results agree with gs_composite_fwd
 *             to float32 rounding: T is a product in another grouping, so a
 *             pixel whose T lands within rounding of 1e-4 may stop one splat
 *             earlier or later, and one that the grouped product puts past
 *             1e-4 but its own walk does not ends with that chunk.
 *             ranges and tile_order are then not read.
 *   part      workspace of gs_composite_part_bytes(cam, capacity) bytes,
 *             16-byte aligned (required with chunks, else unused)
 * Other arguments as gs_composite_fwd. With n_views 1 and ckpt and chunks
 * both NULL this is gs_composite_fwd.
 * ------------------------------------------------------------------- */
gs_status gs_composite_fwd_ex(const gs_camera* cam, int32_t n_views, const uint32_t* ranges,
                              const uint32_t* point_list, const float* xy_depth, const float* conic_op,
                              const float* rgb, const float bg[3], float* image, float* final_T, uint32_t* n_contrib,
                              uint32_t* n_examined, const uint32_t* tile_order, int64_t capacity,
                              float* ckpt, const uint32_t* chunks, void* part, void* stream);

/* gs_composite_part_bytes - bytes of the `part` workspace of
 * gs_composite_fwd_ex for this camera, view count and capacity:
 * (ceil(capacity / 256) + TX TY n_views) * 256 * 20. 0 for invalid
 * arguments. */
size_t gs_composite_part_bytes(const gs_camera* cam, int32_t n_views, int64_t capacity);

/* ---------------------------------------------------------------------
 * gs_composite_bwd_ex - gs_composite_bwd over the work items of the
 * schedule from gs_tile_ranges_ex: 256-entry chunks of the lists, one
 * workgroup per chunk, so that a long list is walked by several workgroups
 * at once (or whole lists, when the schedule says so). Same gradients as
 * gs_composite_bwd
 * ("rigel" README "Backward"), up to float32 rounding: for a chunk that a
 * pixel composited past, the pixel starts from the forward's state at the
 * chunk's end (T from ckpt, and the radiance from behind as image minus the
 * colour accumulated in front: an exact identity that in float32 loses a
 * few bits where little light is left, T near 1e-4); other pixels start
 * from final_T as in gs_composite_bwd.
 *
 *   n_views   as gs_composite_fwd_ex (dL_dimage [n_views][3][H][W]; n
 *             counts the records of the whole stack)
 *   chunks    the schedule gs_tile_ranges_ex wrote for this frame's ranges
 *   capacity  as gs_composite_fwd_ex (the same value)
 *   image     [n_views][3][H][W] the image gs_composite_fwd_ex wrote
 *   ckpt      the checkpoints gs_composite_fwd_ex wrote in the same frame
 *             (may be NULL only when capacity is 0)
 * Other arguments as gs_composite_bwd; every input must come from the same
 * frame (ranges, chunks, the forward's outputs).
 * ------------------------------------------------------------------- */
gs_status gs_composite_bwd_ex(const gs_camera* cam, int32_t n_views, int32_t n, const uint32_t* ranges,
                              const uint32_t* point_list, const uint32_t* chunks, int64_t capacity,
                              const float* xy_depth, const float* conic_op, const float* rgb,
                              const float bg[3], const float* image, const float* final_T,
                              const uint32_t* n_contrib, const float* ckpt, const float* dL_dimage,
                              float* grad_mean2d, float* grad_conic_op, float* grad_rgb, void* stream);

/* ---------------------------------------------------------------------
 * gs_appearance_fwd - colour of every Gaussian from a latent code and the
 * view direction through a small MLP ("rigel" README, "Appearance MLP": an
 * L-float latent concatenated with the unit view direction, an H-wide ReLU
 * layer, a 3-wide sigmoid layer). The result feeds gs_preprocess as rgb_in
 * (the rasterizer never sees how colour was produced).
 *
 *   cam        (host) camera; only campos is used: dir = normalize(mean - campos),
 *              computed as gs_preprocess computes the SH direction
 *   n          number of Gaussians
 *   means      [3][n]
 *   latent     [n_latent][n]
 *   n_latent   L, 1..GS_APP_MAX_LATENT
 *   n_hidden   H, 1..GS_APP_MAX_HIDDEN
 *   weights    packed float32: W1 [H][L+3] (row i = hidden unit i; columns
 *              the latent, then dir x, y, z), b1 [H], W2 [3][H], b2 [3];
 *              H (L+3) + 4H + 3 floats
 *   rgb        out [3][n]: sigmoid(b2 + W2 max(0, b1 + W1 [latent; dir]))
 * z = b1 + W1 x is summed in float32 in input order without fused
 * multiply-add, so which units are active is decided reproducibly.
 * ------------------------------------------------------------------- */
gs_status gs_appearance_fwd(const gs_camera* cam, int32_t n, const float* means, const float* latent,
                            int32_t n_latent, int32_t n_hidden, const float* weights, float* rgb, void* stream);

/* ---------------------------------------------------------------------
 * gs_appearance_bwd - gradients of gs_appearance_fwd ("rigel" README,
 * "Appearance MLP": the latents receive a gradient, the view direction is
 * held constant). With g = dL/drgb:
 *   dy = g s (1 - s);  dz = (W2^T dy) on the active units (z > 0), else 0;
 *   dL/dlatent = W1[:, :L]^T dz;  dW2 = sum dy h^T;  db2 = sum dy;
 *   dW1 = sum dz x^T;  db1 = sum dz  (sums over all n Gaussians).
 * The weight sums are formed per workgroup of 128 Gaussians as dot
 * products and then summed over workgroups in a fixed order: the result is
 * deterministic.
 *
 *   cam, n, means, latent, n_latent, n_hidden, weights: as gs_appearance_fwd
 *   grad_rgb       [3][n] dL/drgb (e.g. grad_rgb_in from gs_preprocess_bwd)
 *   grad_latent    out [n_latent][n]
 *   grad_weights   out, packed as weights (overwritten)
 *   scratch        device workspace of *scratch_bytes bytes (4-byte aligned),
 *                  or NULL to query the size (ceil(n / 128) * (H (L+3) + 4H + 3)
 *                  floats)
 *   scratch_bytes  (host) in: size of scratch; out: required size
 * ------------------------------------------------------------------- */
gs_status gs_appearance_bwd(const gs_camera* cam, int32_t n, const float* means, const float* latent,
                            int32_t n_latent, int32_t n_hidden, const float* weights, const float* grad_rgb,
                            float* grad_latent, float* grad_weights, void* scratch, size_t* scratch_bytes,
                            void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GS_H */
