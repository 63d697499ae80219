// Forward and backward compositing, one 256-lane workgroup (four wave64s)
// per 16x16 tile, one pixel per lane.
//
// Forward: "rigel" README "Rasterization" (block per tile, 256-splat
// shared-memory batches, alpha = min(0.99, o exp(power)), C += c alpha T,
// T *= 1 - alpha, stop below 1e-4, the block exits on a unanimous vote);
// zenn 4.5 (workgroup per tile, cooperative batch staging, composite then
// test the stop threshold); learn-gs "The kernel" (lanes retire by flag and
// keep fetching for the others; the vote is __syncthreads_count).
// Backward: "rigel" README "Backward" (walk back to front from final_T and
// n_contrib, T_i = T_{i+1}/(1-a_i), with what lies behind carried along:
// here as g.R, the upstream gradient dotted with the radiance from behind,
// instead of the colour behind; the two give the same dL/dalpha) and
// "Deliberate differences" (no gradient through a saturated alpha).
//
// MI355X design:
//  * The exponent -0.5 (A dx^2 + C dy^2) - B dx dy is evaluated in fp32 in
//    exactly the written order with no contraction, so it is bit-identical
//    to a host evaluation (this matters: for elongated splats the terms
//    cancel and any other order drifts by more than the image tolerance).
//    exp(power) uses the native base-2 v_exp_f32; only when the resulting
//    alpha lies within a relative 4e-6 of the 1/255 floor (the fast value's
//    error is below 1e-6 there) is the correctly rounded exponential taken
//    (in double), so the skip decision is the exactly defined one.
//  * Both kernels call the same alpha routine, so the backward re-derives
//    exactly the alphas, skips and clamps the forward saw.
//  * Tiles are taken in the order given by tile_order (heaviest list first,
//    from the ranges call), else in workgroup-id order. A launch's length is
//    set by its heaviest tile, which is several times an average slot's
//    share of the work; starting it first lets it overlap everything else.
//    Consecutive workgroup ids go round-robin to the 8 XCDs, so the heavy
//    tiles are spread over all of them (contiguous bands per XCD left some
//    XCDs with most of the work).
//  * Each wave owns an 8 x 8 quadrant of the tile: square strips cull more
//    (splat, strip) pairs than 16 x 4 rows (12% fewer wave iterations on the
//    160k-Gaussian 1080p scene).
//  * Forward: each 16-lane quarter of a wave holds one 4 x 4 block and walks
//    its own list of the staged splats that reach that block, so a wave
//    steps max over its quarters instead of through the union of its four
//    blocks' splats (20% fewer steps at 1080p; the lists are built with
//    ballots per 256-splat batch). Pixels are written in row order
//    after a cross-lane move, and the checkpoints in the backward's order.
//  * Backward: each 16-lane row of a wave holds two pixel rows of its
//    quadrant and the wave walks the union of its blocks' splats. (Per-
//    quarter lists here took 4% fewer VALU instructions but ran slower:
//    every step then waits on a list read before its splat reads, on the
//    heaviest tiles' serial chains.)
//  * Backward: per splat, each wave sums nine per-pixel terms over its 16-lane
//    rows with DPP adds (skipped when no lane contributed) into LDS; the
//    terms are the colour gradient, dL/dpower and its moments (dx, dy, dx^2,
//    dx dy, dy^2 times it), from which the conic, mean and opacity gradients
//    follow once per (splat, tile) (alpha = o G unclamped, so dL/do is the
//    sum of dL/dpower over o). Splats are staged 128 at a time
//    and walked in 32-splat batches; after each batch all
//    256 threads finish it (one output per thread), summing only the
//    partials of waves that wrote them (each wave keeps a mask of the slots
//    it wrote, so the partials need no clearing); one global atomic per value per tile entry
//    lands in the per-Gaussian gradient.
//  * Culling is per 4 x 4 pixel block (see block_mask), exact up to a
//    rounding bound, so a skipped (splat, block) pair changes no result.
//  * Several splats per loop step (three in the forward, two in the
//    backward): their alphas do not depend on one another, so one splat's
//    exponential and reciprocal overlap another's ordered transmittance
//    updates, and the backward's two reductions interleave. A launch lasts as
//    long as its heaviest tiles (lists of 1,000-1,500 splats at 1080p),
//    which end up running almost alone on their compute units; with one
//    splat per step their waves mostly wait on their own latency (measured
//    per workgroup at 1080p: the backward's last 70 of 245 us then ran on
//    under 5% of the workgroup slots).
//  * Long lists in chunks. With a work schedule from the ranges call (see
//    k_tile_schedule) a workgroup takes one 256-entry chunk of a list instead
//    of the whole list, so a long list is walked by several workgroups at
//    once. The forward stores each pixel's (T, C) at every 256-entry
//    boundary; a backward chunk starts a pixel that composited past its end
//    from that state (T, and the radiance from behind as image - C). The
//    scheduled forward composites every chunk from T = 1, then combines the
//    chunks in front of each pixel (T_in *= T_chunk, C += T_in C_chunk) and
//    composites again, splat by splat, the chunk where the pixel stops.
#include "gs_internal.h"

namespace gs {
namespace {

constexpr int kBatch = 256;
static_assert(kChunk == kBatch, "checkpoints are taken at the forward's batch boundaries");
constexpr int kIlpF = 3;  // splats per step of the forward walk
constexpr float kLog2e = 1.4426950408889634f;

// Correctly rounded fp32 exponential (double evaluation, one rounding); the
// rare slow path of splat_alpha, kept out of line.
__device__ __noinline__ float exp_rn(float x) { return (float)exp((double)x); }

// Gaussian weight and alpha of a splat with conic (A, B, C) and opacity o at
// offset (dx, dy) from its centre:
//   power = -0.5 (A dx^2 + C dy^2) - B dx dy,  G = exp(power),
//   alpha = min(0.99, o G),  and oG = o G (unclamped).
// Takes hA = -A/2 and hC = -C/2 (staged once per splat): scaling by a power
// of two commutes with rounding, so (hA dx) dx + (hC dy) dy - (B dx) dy is
// bit-identical to the written order and saves a multiply per pixel.
// In two parts, so that several splats' fast parts can be issued back to
// back behind one wave-uniform test for the rare exact path:
// splat_alpha_fast returns whether alpha lies near the 1/255 floor, and
// splat_alpha_exact recomputes those lanes. splat_alpha does both for one
// splat; it must be called with the whole wave active.
__device__ __forceinline__ bool splat_alpha_fast(float hA, float B, float hC, float o, float dx, float dy,
                                                 float& power, float& G, float& oG, float& alpha) {
    power = ((hA * dx) * dx + (hC * dy) * dy) - (B * dx) * dy;
    G = __builtin_amdgcn_exp2f(power * kLog2e);
    oG = o * G;
    alpha = fminf(kAlphaMax, oG);
    return fabsf(alpha - kAlphaMin) <= kAlphaMin * 4e-6f;  // near the floor: take the exact value
}
__device__ __forceinline__ void splat_alpha_exact(float power, float o, float& G, float& oG, float& alpha) {
    G = exp_rn(power);
    oG = o * G;
    alpha = fminf(kAlphaMax, oG);
}
__device__ __forceinline__ void splat_alpha(float hA, float B, float hC, float o, float dx, float dy,
                                            float& G, float& oG, float& alpha) {
    float power;
    const bool near = splat_alpha_fast(hA, B, hC, o, dx, dy, power, G, oG, alpha);
    if (__builtin_expect(__ballot(near) != 0ull, 0)) {
        if (near) splat_alpha_exact(power, o, G, oG, alpha);
    }
}

// ---- which pixels can a splat reach? ----
//
// A splat can only change a pixel if alpha >= 1/255, i.e. if
// Q(d) = A dx^2 + 2B dx dy + C dy^2 <= 2 ln(255 o): the pixel lies in an
// ellipse. block_mask() marks which of the tile's sixteen 4 x 4 pixel blocks
// that ellipse reaches. For each row of blocks it takes the ellipse's slice
// over the row's y-range: the slice's x-extent is [L, R] with
//   x(dy) = (-B dy -+ sqrt(thr A - det dy^2)) / A,   det = AC - B^2,
// whose right edge is concave and left edge convex in dy, so R (L) is the
// edge at the dy of the ellipse's rightmost (leftmost) point, -+B hx / C,
// clamped into the row's y-range; the blocks of the row whose x-range meets
// [L, R] are kept. The threshold is raised by a bound on the rounding of Q
// in the kernels' fp32 evaluation and of the exponential, and every edge is
// widened by a slack far above this function's own rounding, so a culled
// (splat, block) pair has alpha < 1/255 at every pixel of the block: skipping
// it changes no result. Anything not finite keeps every block.
// Bit 4 by + bx is block (bx, by): pixels x0 + 4 bx .. +3, y0 + 4 by .. +3.
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_sqrt(float x) { return __builtin_amdgcn_sqrtf(x); }
__device__ __forceinline__ float fast_log(float x) { return __logf(x); }

__device__ __forceinline__ uint32_t block_mask(float4 co, float u, float v, int x0, int y0) {
    const float A = co.x, B = co.y, C = co.z, o = co.w;
    if (!(o > 0.0f)) return 0u;  // alpha = o G <= 0 never reaches the floor
    const float rx0 = (float)x0 - u, ry0 = (float)y0 - v;  // tile corner relative to the centre
    const float dxm = fmaxf(fabsf(rx0), fabsf(rx0 + 15.0f)), dym = fmaxf(fabsf(ry0), fabsf(ry0 + 15.0f));
    // 64 ulp of |A| dx^2 + |C| dy^2 + 2|B dx dy| covers the kernels' evaluation of Q
    const float bound = 64.0f * 5.96e-8f * (fabsf(A) + fabsf(C) + 2.0f * fabsf(B));
    const float thr = 2.0f * fast_log(255.0f * o) * (1.0f + 1e-5f) + 1e-3f + bound * (dxm * dxm + dym * dym);
    if (thr <= 0.0f) return 0u;  // Q >= 0 > thr everywhere
    const float det = A * C - B * B;
    if (!(det > 0.0f && A > 0.0f && C > 0.0f && thr < 3.0e38f)) return 0xFFFFu;
    const float idet = fast_rcp(det), iA = fast_rcp(A);
    const float hy = fast_sqrt(thr * A * idet);  // half-extents of the ellipse
    const float hx = fast_sqrt(thr * C * idet);
    const float ydr = -B * hx * fast_rcp(C);     // dy of the rightmost point; the leftmost is at -ydr
    const float slack = 1e-2f + 1e-4f * (hx + hy);
    const float thrA = thr * A;
    uint32_t mask = 0u;
#pragma unroll
    for (int by = 0; by < 4; ++by) {
        const float y0r = ry0 + (float)(4 * by);
        const float lo = fmaxf(y0r, -hy), hi = fminf(y0r + 3.0f, hy);
        if (lo > hi + slack) continue;  // the row's y-range misses the ellipse (false on NaN)
        const float yr = fminf(fmaxf(ydr, lo), hi);
        const float yl = fminf(fmaxf(-ydr, lo), hi);
        const float R = (-B * yr + fast_sqrt(fmaxf(0.0f, thrA - det * yr * yr))) * iA + slack;
        const float L = (-B * yl - fast_sqrt(fmaxf(0.0f, thrA - det * yl * yl))) * iA - slack;
        // block bx spans [rx0 + 4 bx, rx0 + 4 bx + 3]; keep bx in [ceil((L - rx0 - 3) / 4), floor((R - rx0) / 4)]
        const float flo = fmaxf(ceilf((L - rx0 - 3.0f) * 0.25f), 0.0f);   // NaN -> 0
        const float fhi = fminf(floorf((R - rx0) * 0.25f), 3.0f);         // NaN -> 3
        if (flo <= fhi) mask |= ((2u << (int)fhi) - (1u << (int)flo)) << (4 * by);
    }
    return mask;
}

// Pixel of a lane within its 16 x 16 tile: wave w owns the 8 x 8 quadrant
// (w & 1, w >> 1), and quarter r = lane / 16 of the wave the 4 x 4 block
// (r & 1, r >> 1) of that quadrant, row by row.
__device__ __forceinline__ int lane_px(int wave, int lane) {
    return 8 * (wave & 1) + 4 * ((lane >> 4) & 1) + (lane & 3);
}
__device__ __forceinline__ int lane_py(int wave, int lane) {
    return 8 * (wave >> 1) + 4 * (lane >> 5) + ((lane >> 2) & 3);
}
// The blocks of the backward's wave w: its 8 x 8 quadrant (blocks
// 2 (w & 1) .. +1 of rows 2 (w >> 1) .. +1).
__device__ __forceinline__ uint32_t quadrant_blocks(int w) {
    return 0x33u << (2 * (w & 1) + 8 * (w >> 1));
}
// block_mask bit of quarter r of wave w (bit 4 by + bx for block (bx, by)).
__device__ __forceinline__ uint32_t quarter_bit(int w, int r) {
    return 1u << (4 * (2 * (w >> 1) + (r >> 1)) + 2 * (w & 1) + (r & 1));
}
// Per-pixel image data is read and written in row order instead (lane L of
// a wave: pixel (L & 7, L >> 3) of its quadrant, 8 consecutive pixels per 8
// lanes), then moved across lanes: a 16-lane quarter's 4 x 4 block spans four
// rows, so block-order accesses touch twice as many cache lines per group of
// lanes as row-order ones. row_lane: the row-order lane of this lane's pixel;
// quarter_lane: the lane that holds row-order lane L's pixel.
__device__ __forceinline__ int row_lane(int lane) {
    return (4 * (lane >> 5) + ((lane >> 2) & 3)) * 8 + 4 * ((lane >> 4) & 1) + (lane & 3);
}
__device__ __forceinline__ int quarter_lane(int L) {
    const int qx = L & 7, qy = L >> 3;
    return 16 * (2 * (qy >> 2) + (qx >> 2)) + 4 * (qy & 3) + (qx & 3);
}

// A stack of views shares one tile grid: view b is the band of tile rows
// [b TYb, b TYb + TYb), and its pixels keep their own coordinates (the
// splat records of a view are in that view's pixels). Tile column, row
// within the band, and band of a tile id.
struct TileAt {
    int tx, ty, band;
};
__device__ __forceinline__ TileAt tile_at(int tile, int TX, int TYb) {
    const int row = tile / TX;
    const int band = row / TYb;
    return {tile - row * TX, row - band * TYb, band};
}

// Staged records are addressed by byte offset (slot x 16) from the quarter
// lists. Slot kBatch holds a sentinel record (conic 0, opacity 0): its alpha
// is 0, below the floor, so a lane that reads it changes nothing. Lists are
// built for kHalf staged slots at a time: the whole batch (all four waves'
// lists, u16 entries, and the staged records take 20.9 KB, seven workgroups
// per CU; lists over 128-slot halves measured 0.6% slower per frame).
constexpr int kHalf = kBatch;
constexpr int kListCap = kHalf + kIlpF + 1;  // a list, its kIlpF sentinel entries, padding
constexpr uint32_t kSentF = (uint32_t)kBatch * 16u;

template <typename V>
__device__ __forceinline__ const V& at_byte(const V* base, uint32_t off) {
    return *reinterpret_cast<const V*>(reinterpret_cast<const char*>(base) + off);
}

// Stages list entries [base, min(base + kBatch, end)) into LDS, one per
// thread: the conic with -1/2 folded in, the centre and colour, and the
// 4 x 4 blocks of the tile the splat reaches (none for slots past the end).
__device__ __forceinline__ void fwd_stage(uint32_t base, uint32_t end, int tid, int x0, int y0,
                                          const uint32_t* __restrict__ point_list,
                                          const float4* __restrict__ xy_depth, const float4* __restrict__ conic_op,
                                          const float4* __restrict__ rgb, float4* s_conic, float4* s_xyc,
                                          float4* s_bl) {
    const uint32_t j = base + (uint32_t)tid;
    if (j < end) {
        const uint32_t g = point_list[j];
        const float4 xy = xy_depth[g];
        const float4 co = conic_op[g];
        const float4 c = rgb[g];
        s_conic[tid] = make_float4(-0.5f * co.x, co.y, -0.5f * co.z, co.w);
        s_xyc[tid] = make_float4(xy.x, xy.y, c.x, c.y);
        s_bl[tid] = make_float4(c.z, __uint_as_float(block_mask(co, xy.x, xy.y, x0, y0)), 0.0f, 0.0f);
    } else {
        // a slot past the end is never walked: only its (empty) block bits are read
        reinterpret_cast<float*>(s_bl + tid)[1] = 0.0f;
    }
}

// The sentinel record at slot `slot` (called by one thread).
__device__ __forceinline__ void stage_sentinel(int slot, float4* s_conic, float4* s_xyc, float4* s_third) {
    s_conic[slot] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    s_xyc[slot] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    s_third[slot] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
}

// Composites the cnt staged splats (list positions pos0 ..) front to back
// into this lane's (T, C, last). A lane whose T is below the stop threshold
// has stopped and changes nothing. All 64 lanes of the wave take part.
// Each 16-lane quarter walks only the splats that reach its 4 x 4 block:
// per kHalf staged slots, the wave writes each quarter's list of them (in
// list order) to s_list (this wave's four lists, kListCap entries each),
// then steps through the four lists side by side, kIlpF entries per step,
// until every quarter has run out or stopped; a quarter past its end reads
// sentinel entries.
__device__ __forceinline__ void fwd_walk(int cnt, uint32_t pos0, int wave, int lane, float fx, float fy,
                                         const float4* s_conic, const float4* s_xyc, const float4* s_bl,
                                         uint16_t* s_list, float& T, float& C0, float& C1, float& C2,
                                         uint32_t& last) {
    const int rq = lane >> 4;  // this lane's quarter
    uint16_t* const my_list = s_list + rq * kListCap;
    for (int h = 0; h < cnt; h += kHalf) {
        const uint64_t going = __ballot(T >= kTStop);
        if (going == 0ull) return;
        uint32_t n[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < kHalf; c += 64) {
            if (h + c < cnt) {
                const int slot = h + c + lane;  // < kBatch; past the end its block mask is empty
                const uint32_t bits = __float_as_uint(s_bl[slot].y);
                const uint16_t entry = (uint16_t)(slot * 16);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (((going >> (16 * r)) & 0xFFFFull) != 0ull) {  // quarter r has a pixel going
                        const bool in = (bits & quarter_bit(wave, r)) != 0u;
                        const uint64_t m = __ballot(in);
                        const uint32_t pos =
                            __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, n[r]));
                        if (in) s_list[r * kListCap + pos] = entry;
                        n[r] += (uint32_t)__popcll(m);
                    }
                }
            }
        }
        const uint32_t nl = rq == 0 ? n[0] : rq == 1 ? n[1] : rq == 2 ? n[2] : n[3];
        if ((lane & 15) < kIlpF) my_list[nl + (uint32_t)(lane & 15)] = (uint16_t)kSentF;
        const uint32_t nmax = max(max(n[0], n[1]), max(n[2], n[3]));
        uint32_t lastl = kSentF;  // byte offset of this half's last splat composited, if any
        for (uint32_t p = 0; p < nmax; p += kIlpF) {
            if (__ballot(T >= kTStop && p < nl) == 0ull) break;
            const uint32_t pc = min(p, nl);
            // kIlpF splats per step: independent alphas, then the ordered updates
            uint32_t e[kIlpF];
#pragma unroll
            for (int i = 0; i < kIlpF; ++i) e[i] = my_list[pc + (uint32_t)i];
            float4 co[kIlpF], xc[kIlpF];
            float cb[kIlpF], pw[kIlpF], G[kIlpF], oG[kIlpF], alpha[kIlpF];
            bool near[kIlpF];
            bool any_near = false;
#pragma unroll
            for (int i = 0; i < kIlpF; ++i) {
                co[i] = at_byte(s_conic, e[i]);
                xc[i] = at_byte(s_xyc, e[i]);
                cb[i] = at_byte(s_bl, e[i]).x;
            }
#pragma unroll
            for (int i = 0; i < kIlpF; ++i) {
                near[i] = splat_alpha_fast(co[i].x, co[i].y, co[i].z, co[i].w, fx - xc[i].x, fy - xc[i].y, pw[i],
                                           G[i], oG[i], alpha[i]);
                any_near = any_near || near[i];
            }
            if (__builtin_expect(__ballot(any_near) != 0ull, 0)) {
#pragma unroll
                for (int i = 0; i < kIlpF; ++i)
                    if (near[i]) splat_alpha_exact(pw[i], co[i].w, G[i], oG[i], alpha[i]);
            }
#pragma unroll
            for (int i = 0; i < kIlpF; ++i) {
                // branch-free update; stopped lanes, sentinels and alphas below
                // the floor change nothing (w = 0). T (1 - alpha) is taken as
                // T - alpha T, the weight already at hand: one instruction
                // instead of three, within an ulp of the product.
                const bool use = T >= kTStop && alpha[i] >= kAlphaMin;
                const float w = use ? alpha[i] * T : 0.0f;
                C0 = __builtin_fmaf(xc[i].z, w, C0);
                C1 = __builtin_fmaf(xc[i].w, w, C1);
                C2 = __builtin_fmaf(cb[i], w, C2);
                T = T - w;
                lastl = use ? e[i] : lastl;
            }
        }
        if (lastl != kSentF) last = pos0 + (lastl >> 4) + 1u;
    }
}

__device__ __forceinline__ void fwd_write(int W, int H, int px, int py, float3 bg, float T, float C0, float C1,
                                          float C2, uint32_t last, uint32_t examined, float* __restrict__ image,
                                          float* __restrict__ final_T, uint32_t* __restrict__ n_contrib,
                                          uint32_t* __restrict__ n_examined) {
    const size_t p = (size_t)py * W + px;
    const size_t plane = (size_t)W * H;
    image[p] = __builtin_fmaf(T, bg.x, C0);
    image[plane + p] = __builtin_fmaf(T, bg.y, C1);
    image[2 * plane + p] = __builtin_fmaf(T, bg.z, C2);
    final_T[p] = T;
    n_contrib[p] = last;
    if (n_examined) n_examined[p] = examined;
}

// Row of the chunk partials of chunk b of a list (start, len): the
// checkpoint slot of the chunk's end boundary, or, for the list's last
// chunk, slot n_slots + tile.
__device__ __forceinline__ size_t part_row(uint32_t start, uint32_t len, uint32_t b, uint32_t n_slots, int tile) {
    const uint32_t end_rel = (b + 1u) * (uint32_t)kChunk;
    return end_rel < len ? (size_t)((start + end_rel) / kChunk) : (size_t)n_slots + (size_t)tile;
}

// Forward compositing. Whole lists (kItems false): workgroup i takes tile
// tile_order[i]. Scheduled (kItems true): workgroup i takes work item i of
// `chunks` (see the backward): a whole list is composited as above; a chunk
// is composited from T = 1 and C = 0 with the stop rule applied to that
// local T, and its per-pixel (T, C, last) land in part / part_last for
// k_composite_fwd_resolve, which writes the outputs of its pixels.
template <bool kItems>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(7, 7))) void k_composite_fwd(
    const int W, const int H, const int TX, const int TYb, const uint32_t* __restrict__ ranges,
    const uint32_t* __restrict__ point_list, const float4* __restrict__ xy_depth,
    const float4* __restrict__ conic_op, const float4* __restrict__ rgb, const float3 bg,
    float* __restrict__ image, float* __restrict__ final_T, uint32_t* __restrict__ n_contrib,
    uint32_t* __restrict__ n_examined, const uint32_t* __restrict__ tile_order, float4* __restrict__ ckpt,
    const uint32_t ckpt_slots, const uint32_t* __restrict__ chunks, const uint32_t n_tiles, const uint32_t n_slots,
    float4* __restrict__ part, uint32_t* __restrict__ part_last) {
    __shared__ float4 s_conic[kBatch + 1];  // -A/2, B, -C/2, opacity (slot kBatch: the sentinel)
    __shared__ float4 s_xyc[kBatch + 1];    // u, v, r, g
    __shared__ float4 s_bl[kBatch + 1];     // b, live blocks (as bits), -, -: one address with the two above
    __shared__ uint16_t s_list[4][4][kListCap];  // per wave, per quarter: staged slots to walk

    int tile;
    uint32_t start, end, base0, len = 0, chunk = kWholeList;
    if (kItems) {
        const uint32_t count = chunks[0];
        const uint4 item = reinterpret_cast<const uint4*>(chunks + 4)[blockIdx.x];
        if (blockIdx.x >= count || item.x >= n_tiles) return;
        tile = (int)item.x;
        chunk = item.y;
        start = item.z;
        len = item.w;
        end = start + len;
        base0 = start;
        if (chunk != kWholeList) {
            base0 = start + chunk * (uint32_t)kChunk;
            end = min(end, base0 + (uint32_t)kChunk);
        }
    } else {
        tile = tile_order ? (int)tile_order[blockIdx.x] : (int)blockIdx.x;
        start = ranges[2 * tile];
        end = ranges[2 * tile + 1];
        base0 = start;
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const TileAt ta = tile_at(tile, TX, TYb);
    const int tx = ta.tx, ty = ta.ty;
    {  // this view's outputs
        const size_t view_px = (size_t)W * H;
        image += (size_t)ta.band * 3 * view_px;
        final_T += (size_t)ta.band * view_px;
        n_contrib += (size_t)ta.band * view_px;
        if (n_examined) n_examined += (size_t)ta.band * view_px;
    }
    const int px = tx * kTile + lane_px(wave, lane);
    const int py = ty * kTile + lane_py(wave, lane);
    const bool inside = px < W && py < H;
    const float fx = (float)px, fy = (float)py;
    // this pixel's slot in a checkpoint row: the backward's thread for it
    const int ck_idx = wave * 64 + row_lane(lane);

    // A pixel has stopped exactly when its transmittance is below the stop
    // threshold (T only decreases, and compositing ends at the first splat
    // that takes it there), so no separate flag is carried. A lane outside
    // the image starts stopped (T = 0; it writes nothing).
    float T = inside ? 1.0f : 0.0f, C0 = 0.0f, C1 = 0.0f, C2 = 0.0f;
    uint32_t last = 0;
    if (tid == 0) stage_sentinel(kBatch, s_conic, s_xyc, s_bl);  // seen after the first staging barrier

    for (uint32_t base = base0; base < end; base += kBatch) {
        // the state in front of this batch, for a backward chunk that ends
        // here; boundaries inside one list are 256 apart and those of the next
        // list lie more than 256 beyond, so base / 256 is a slot of its own
        if (chunk == kWholeList && base != start && base / kChunk < ckpt_slots)
            ckpt[(size_t)(base / kChunk) * kChunk + ck_idx] = make_float4(T, C0, C1, C2);
        if (__syncthreads_count(T < kTStop) == 256) break;
        fwd_stage(base, end, tid, tx * kTile, ty * kTile, point_list, xy_depth, conic_op, rgb, s_conic, s_xyc, s_bl);
        __syncthreads();
        fwd_walk((int)min((uint32_t)kBatch, end - base), base - start, wave, lane, fx, fy, s_conic, s_xyc, s_bl,
                 &s_list[wave][0][0], T, C0, C1, C2, last);
    }

    if (kItems && chunk != kWholeList) {
        const size_t r = part_row(start, len, chunk, n_slots, tile) * kChunk + tid;
        part[r] = make_float4(T, C0, C1, C2);
        part_last[r] = last;
    } else {
        // written in row order: each lane takes the state of row-order pixel
        // `lane` from the lane that composited it. A pixel that stopped
        // examined up to its last contributor; one that did not examined the
        // whole list.
        const int src = quarter_lane(lane);
        const float Tr = __shfl(T, src, 64), C0r = __shfl(C0, src, 64), C1r = __shfl(C1, src, 64),
                    C2r = __shfl(C2, src, 64);
        const uint32_t lastr = (uint32_t)__shfl((int)last, src, 64);
        const int rx = tx * kTile + 8 * (wave & 1) + (lane & 7), ry = ty * kTile + 8 * (wave >> 1) + (lane >> 3);
        if (rx < W && ry < H)
            fwd_write(W, H, rx, ry, bg, Tr, C0r, C1r, C2r, lastr, Tr < kTStop ? lastr : end - start, image, final_T,
                      n_contrib, n_examined);
    }
}

// Outputs of the pixels whose lists were composited in chunks. Workgroup i
// takes work item i of `chunks` when it is chunk b of a list (whole lists
// are done): each pixel combines the partials of chunks 0 .. b-1 front to
// back (T_in *= T_j, C += T_in C_j, in list order). A pixel whose
// transmittance crosses the stop threshold inside an earlier chunk belongs
// to that chunk's workgroup. A pixel still going stores the checkpoint at
// the chunk's start; if the chunk's partial takes it below the threshold it
// is composited again through the chunk from (T_in, C), splat by splat as
// the whole-list walk does, stopping where that walk stops; if not and this
// is the list's last chunk, the combined state is final.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(7, 7))) void k_composite_fwd_resolve(
    const int W, const int H, const int TX, const int TYb, const uint32_t* __restrict__ point_list,
    const float4* __restrict__ xy_depth, const float4* __restrict__ conic_op, const float4* __restrict__ rgb,
    const float3 bg, float* __restrict__ image, float* __restrict__ final_T, uint32_t* __restrict__ n_contrib,
    uint32_t* __restrict__ n_examined, float4* __restrict__ ckpt, const uint32_t* __restrict__ chunks,
    const uint32_t n_tiles, const uint32_t n_slots, const float4* __restrict__ part,
    const uint32_t* __restrict__ part_last) {
    __shared__ float4 s_conic[kBatch + 1];
    __shared__ float4 s_xyc[kBatch + 1];
    __shared__ float4 s_bl[kBatch + 1];
    __shared__ uint16_t s_list[4][4][kListCap];

    const uint32_t count = chunks[0];
    const uint4 item = reinterpret_cast<const uint4*>(chunks + 4)[blockIdx.x];
    if (blockIdx.x >= count || item.x >= n_tiles || item.y == kWholeList) return;
    const int tile = (int)item.x;
    const uint32_t b = item.y, start = item.z, len = item.w;
    const uint32_t lo = b * (uint32_t)kChunk, hi = min(lo + (uint32_t)kChunk, len);
    const bool last_chunk = hi == len;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const TileAt ta = tile_at(tile, TX, TYb);
    const int tx = ta.tx, ty = ta.ty;
    {  // this view's outputs
        const size_t view_px = (size_t)W * H;
        image += (size_t)ta.band * 3 * view_px;
        final_T += (size_t)ta.band * view_px;
        n_contrib += (size_t)ta.band * view_px;
        if (n_examined) n_examined += (size_t)ta.band * view_px;
    }
    const int px = tx * kTile + lane_px(wave, lane);
    const int py = ty * kTile + lane_py(wave, lane);
    const bool inside = px < W && py < H;
    const float fx = (float)px, fy = (float)py;
    // this pixel's slot in a checkpoint row: the backward's thread for it
    const int ck_idx = wave * 64 + row_lane(lane);

    float T = 1.0f, C0 = 0.0f, C1 = 0.0f, C2 = 0.0f;
    uint32_t last = 0;
    bool alive = inside;
    for (uint32_t j = 0; j < b; ++j) {
        if (alive) {
            const size_t r = part_row(start, len, j, n_slots, tile) * kChunk + tid;
            const float4 q = part[r];
            const uint32_t lj = part_last[r];
            const float Tn = T * q.x;
            if (Tn < kTStop) {
                alive = false;  // stops inside chunk j
            } else {
                C0 = __builtin_fmaf(T, q.y, C0);
                C1 = __builtin_fmaf(T, q.z, C1);
                C2 = __builtin_fmaf(T, q.w, C2);
                T = Tn;
                last = lj != 0u ? lj : last;
            }
        }
    }
    if (alive && b != 0u && ckpt && (start + lo) / kChunk < n_slots)
        ckpt[(size_t)((start + lo) / kChunk) * kChunk + ck_idx] = make_float4(T, C0, C1, C2);
    bool walk = false;
    if (alive) {
        const size_t r = part_row(start, len, b, n_slots, tile) * kChunk + tid;
        const float4 q = part[r];
        const uint32_t lb = part_last[r];
        const float Tn = T * q.x;
        if (Tn < kTStop) {
            walk = true;
        } else if (last_chunk) {
            fwd_write(W, H, px, py, bg, Tn, __builtin_fmaf(T, q.y, C0), __builtin_fmaf(T, q.z, C1),
                      __builtin_fmaf(T, q.w, C2), lb != 0u ? lb : last, len, image, final_T, n_contrib, n_examined);
        }
    }
    if (__syncthreads_or(walk)) {
        fwd_stage(start + lo, start + hi, tid, tx * kTile, ty * kTile, point_list, xy_depth, conic_op, rgb, s_conic,
                  s_xyc, s_bl);
        if (tid == 0) stage_sentinel(kBatch, s_conic, s_xyc, s_bl);
        __syncthreads();
        float Tw = walk ? T : 0.0f;  // only these lanes composite
        fwd_walk((int)(hi - lo), lo, wave, lane, fx, fy, s_conic, s_xyc, s_bl, &s_list[wave][0][0], Tw, C0, C1, C2,
                 last);
        // stopped here (or, if rounding kept it just above the threshold,
        // ended with this chunk)
        if (walk) fwd_write(W, H, px, py, bg, Tw, C0, C1, C2, last, Tw < kTStop ? last : hi, image, final_T, n_contrib,
                            n_examined);
    }
}

// x plus the value of x that DPP control kCtrl moves into this lane (lane
// permutes within a row of 16). Must be called with all 64 lanes active.
template <int kCtrl>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, true));
}

template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, true));
}

// Transpose-reduce of nine per-lane values over each 16-lane row into one
// register: lane j of a row ends with the row sum of value j for j < 8, and
// lanes 8..15 with that of value 8. Each merge step pairs every lane with a
// partner whose lane bit b differs (quad_perm for bits 0 and 1, a rotation of
// the row by 4 and by 8 for bits 2 and 3: both flip the bit); a lane keeps
// the half of its values that its bit selects and adds its partner's copy of
// the same values, so the live values halve while the lanes summed double.
// Value 8 is summed over half rows first and enters at the last step. 27
// instructions, against 26 for two four-value transposes and a row sum into
// three registers. b0..b3: lane bits 0..3. All 64 lanes must be active.
__device__ __forceinline__ float transpose_row_sum9(float a0, float a1, float a2, float a3, float a4, float a5,
                                                   float a6, float a7, float a8, bool b0, bool b1, bool b2,
                                                   bool b3) {
    const float p01 = (b0 ? a1 : a0) + dpp_mov<0xB1>(b0 ? a0 : a1);  // quad_perm [1,0,3,2]
    const float p23 = (b0 ? a3 : a2) + dpp_mov<0xB1>(b0 ? a2 : a3);
    const float p45 = (b0 ? a5 : a4) + dpp_mov<0xB1>(b0 ? a4 : a5);
    const float p67 = (b0 ? a7 : a6) + dpp_mov<0xB1>(b0 ? a6 : a7);
    const float qa = (b1 ? p23 : p01) + dpp_mov<0x4E>(b1 ? p01 : p23);  // quad_perm [2,3,0,1]
    const float qb = (b1 ? p67 : p45) + dpp_mov<0x4E>(b1 ? p45 : p67);
    const float r = (b2 ? qb : qa) + dpp_mov<0x124>(b2 ? qa : qb);      // row_ror:4
    float h8 = dpp_add<0xB1>(a8);
    h8 = dpp_add<0x4E>(h8);
    h8 = dpp_add<0x141>(h8);                                             // row_half_mirror
    return (b3 ? h8 : r) + dpp_mov<0x128>(b3 ? r : h8);                  // row_ror:8
}

__device__ __forceinline__ void atomic_add_nz(float* p, float v) {
    if (v != 0.0f) unsafeAtomicAdd(p, v);
}

// Clears the three gradient arrays (n x 2, n x 4, n x 4 floats) in one launch.
__global__ void k_zero_grads(float2* __restrict__ gm, float4* __restrict__ gc, float4* __restrict__ gr, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        gm[i] = make_float2(0.f, 0.f);
        gc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        gr[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

// Per (splat, wave) the nine terms are summed over each 16-lane row with
// DPP; the four row sums of each wave go to LDS (16 partials per splat).
// Term t of row slot s is stored at slot s ^ part_swizzle(t), so terms 0..7
// of one wave's four rows fall in 32 different banks.
constexpr int kBwdBatch = 32;
// Splats staged per round, walked in batches of kBwdBatch: the gathers of a
// round (list entry, then the splat's records) are two dependent memory
// round trips, paid once per round. The heaviest tile bounds the launch and
// its workgroup runs nearly alone, so that latency is on its critical path.
constexpr int kBwdStage = 128;
constexpr int kParts = 16;  // 4 waves x 4 rows
__host__ __device__ constexpr int part_swizzle(int t) { return t < 8 ? ((t & 2) << 1) | ((t & 4) << 1) : 0; }

// Work items. Whole lists (kChunked false): item i is tile tile_order[i].
// Scheduled (kChunked true): item i is entry i of the schedule `chunks` (a
// count, then (tile, chunk b, list start, list length)), chunk b covering
// tile-relative list positions [256 b, 256 b + 256), or the whole list when
// b is kWholeList. A chunk starts each pixel from the final state when the
// pixel composited nothing past the chunk's end, else from the forward's
// checkpoint there: T, and g.R = g.(image - accumulated colour).
template <bool kChunked>
__global__ __launch_bounds__(256) void k_composite_bwd(
    const int W, const int H, const int TX, const int TYb, const uint32_t* __restrict__ ranges,
    const uint32_t* __restrict__ point_list, const float4* __restrict__ xy_depth,
    const float4* __restrict__ conic_op, const float4* __restrict__ rgb, const float3 bg,
    const float* __restrict__ final_T, const uint32_t* __restrict__ n_contrib,
    const float* __restrict__ dL_dimage, float* __restrict__ grad_mean2d,
    float* __restrict__ grad_conic_op, float* __restrict__ grad_rgb, const uint32_t* __restrict__ tile_order,
    const uint32_t* __restrict__ chunks, const uint32_t n_slots, const uint32_t n_tiles,
    const float4* __restrict__ ckpt, const float* __restrict__ image) {
    __shared__ float4 s_conic[kBwdStage];  // -A/2, B, -C/2, opacity
    __shared__ float4 s_xyc[kBwdStage];    // u, v, r, g
    __shared__ float4 s_aux[kBwdStage];    // b, Gaussian id, -, -: one address with the two above
    __shared__ uint32_t s_live[kBwdStage];
    __shared__ __align__(16) float s_part[kBwdBatch][9][kParts];  // per-row partial sums
    __shared__ uint32_t s_wmask[4];  // the batch's slots whose partials wave w wrote (bit k: slot k)
    __shared__ uint32_t s_maxnc[4];

    int tile;
    int lo = 0;  // first tile-relative position of this item
    bool whole_item = true;
    uint32_t start, len;
    if (kChunked) {
        const uint32_t count = chunks[0];
        const uint4 item = reinterpret_cast<const uint4*>(chunks + 4)[blockIdx.x];
        if (blockIdx.x >= count || item.x >= n_tiles) return;
        tile = (int)item.x;
        whole_item = item.y == kWholeList;
        lo = whole_item ? 0 : (int)(item.y * (uint32_t)kChunk);
        start = item.z;
        len = item.w;
    } else {
        tile = tile_order ? (int)tile_order[blockIdx.x] : (int)blockIdx.x;
        start = ranges[2 * tile];
        len = ranges[2 * tile + 1] - start;
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const bool lane_b0 = (lane & 1) != 0, lane_b1 = (lane & 2) != 0, lane_b2 = (lane & 4) != 0,
               lane_b3 = (lane & 8) != 0;
    const TileAt ta = tile_at(tile, TX, TYb);
    const int tx = ta.tx, ty = ta.ty;
    {  // this view's pixels
        const size_t view_px = (size_t)W * H;
        final_T += (size_t)ta.band * view_px;
        n_contrib += (size_t)ta.band * view_px;
        dL_dimage += (size_t)ta.band * 3 * view_px;
        if (image) image += (size_t)ta.band * 3 * view_px;
    }
    const int px = tx * kTile + 8 * (wave & 1) + (lane & 7);
    const int py = ty * kTile + 8 * (wave >> 1) + (lane >> 3);
    const uint32_t qblocks = quadrant_blocks(wave);
    // the one LDS store per (splat, wave): lane j <= 8 of each row writes its
    // row's sum of term j; which slots a wave wrote is kept in s_wmask
    const int j16 = lane & 15;
    const int my_term = min(j16, 8);
    const bool store_lane = j16 <= 8;
    float* const store_base = &s_part[0][my_term][(wave * 4 + (lane >> 4)) ^ part_swizzle(my_term)];
    constexpr int store_stride = 9 * kParts;
    const bool inside = px < W && py < H;
    const float fx = (float)px, fy = (float)py;
    // g.R: the upstream gradient dotted with the radiance from behind the
    // splats walked so far (their c alpha T, plus the background's T_final
    // bg). With it dL/dalpha_j = T_j (g.c_j) - (g.R_j) / (1 - alpha_j): the
    // colour behind splat j is R_j / T_(j+1), and T_(j+1) = T_j (1 - alpha_j).
    const int hi_item = whole_item ? (int)len : min(lo + kChunk, (int)len);  // this item walks [lo, hi_item)
    float T = 1.0f, g0 = 0.0f, g1 = 0.0f, g2 = 0.0f, gR = 0.0f;
    uint32_t nc = 0;
    if (inside) {
        const size_t p = (size_t)py * W + px;
        const size_t plane = (size_t)W * H;
        T = final_T[p];
        nc = min(n_contrib[p], len);  // never walk past the tile's list
        g0 = dL_dimage[p];
        g1 = dL_dimage[plane + p];
        g2 = dL_dimage[2 * plane + p];
        gR = T * __builtin_fmaf(g2, bg.z, __builtin_fmaf(g1, bg.y, g0 * bg.x));
        const uint32_t ck_slot = (start + (uint32_t)hi_item) / kChunk;
        if (kChunked && (int)nc > hi_item && ck_slot < n_slots) {
            // composited past the chunk: resume from the forward's state there
            const float4 ck = ckpt[(size_t)ck_slot * kChunk + tid];
            T = ck.x;
            gR = __builtin_fmaf(g2, image[2 * plane + p] - ck.w,
                                __builtin_fmaf(g1, image[plane + p] - ck.z, g0 * (image[p] - ck.y)));
        }
    }

    // per-wave and per-tile maximum of n_contrib
    uint32_t wmax = nc;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) wmax = max(wmax, (uint32_t)__shfl_xor((int)wmax, off, 64));
    if (lane == 0) s_maxnc[wave] = wmax;
    __syncthreads();
    const int maxnc = (int)max(max(s_maxnc[0], s_maxnc[1]), max(s_maxnc[2], s_maxnc[3]));
    const int wave_maxnc = (int)wmax;

    for (int send = min(maxnc, hi_item); send > lo; send -= kBwdStage) {  // rounds, back to front
        const int sstart = send - kBwdStage > lo ? send - kBwdStage : lo;
        __syncthreads();  // the previous round is fully consumed
        if (tid < send - sstart) {
            const uint32_t g = point_list[start + sstart + tid];
            const float4 xy = xy_depth[g];
            const float4 co = conic_op[g];
            const float4 c = rgb[g];
            s_conic[tid] = make_float4(-0.5f * co.x, co.y, -0.5f * co.z, co.w);
            s_xyc[tid] = make_float4(xy.x, xy.y, c.x, c.y);
            s_aux[tid] = make_float4(c.z, __uint_as_float(g), 0.0f, 0.0f);
            s_live[tid] = block_mask(co, xy.x, xy.y, tx * kTile, ty * kTile);
        }
        for (int bend = send; bend > sstart; bend -= kBwdBatch) {  // batches of the round
            const int bstart = bend - kBwdBatch > sstart ? bend - kBwdBatch : sstart;
            const int cnt = bend - bstart;
            const int off = bstart - sstart;  // staging slot of this batch's slot 0
            __syncthreads();  // staged, and the previous batch's partials are consumed

            // live splats of this wave below its largest n_contrib, walked back to front
            static_assert(kBwdBatch <= 64, "one 64-bit live mask");
            const int ls = min(off + lane, kBwdStage - 1);  // (lanes past cnt read a valid slot, unused)
            uint64_t mk = __ballot(lane < cnt && bstart + lane < wave_maxnc && (s_live[ls] & qblocks) != 0u);
            const int ncb = (int)nc - bstart;  // this lane uses slot k only if k < ncb
            static_assert(kBwdBatch <= 32, "one 32-bit mask of stored slots");
            uint32_t stored = 0u;  // slots whose partials this wave wrote (wave-uniform)
            // Two splats per step: their alphas are independent, so the second's
            // exponential and reciprocal overlap the first's updates, and the two
            // reductions interleave. A launch lasts as long as its heaviest tiles,
            // which end up running nearly alone on their compute units, where a
            // single splat per step leaves the wave waiting on its own latency.
            while (mk != 0ull) {
                const int k1 = 63 - __clzll((long long)mk);
                mk &= ~(1ull << k1);
                const bool two = mk != 0ull;
                const int k2 = two ? 63 - __clzll((long long)mk) : k1;
                mk &= ~(1ull << k2);
                const float4 co1 = s_conic[off + k1], xc1 = s_xyc[off + k1];
                const float4 co2 = s_conic[off + k2], xc2 = s_xyc[off + k2];
                const float cb1 = s_aux[off + k1].x, cb2 = s_aux[off + k2].x;
                const float dx1 = fx - xc1.x, dy1 = fy - xc1.y;
                const float dx2 = fx - xc2.x, dy2 = fy - xc2.y;
                float G1, oG1, alpha1, G2, oG2, alpha2;
                splat_alpha(co1.x, co1.y, co1.z, co1.w, dx1, dy1, G1, oG1, alpha1);
                splat_alpha(co2.x, co2.y, co2.z, co2.w, dx2, dy2, G2, oG2, alpha2);
                // branch-free: a lane past its n_contrib or below the floor
                // takes alpha 0, so T / (1 - 0) = T exactly and it adds nothing
                const bool use1 = k1 < ncb && alpha1 >= kAlphaMin;
                const bool use2 = two && k2 < ncb && alpha2 >= kAlphaMin;
                const float a1 = use1 ? alpha1 : 0.0f, a2 = use2 ? alpha2 : 0.0f;
                const float rinv1 = __builtin_amdgcn_rcpf(1.0f - a1);
                const float rinv2 = __builtin_amdgcn_rcpf(1.0f - a2);
                float t1[9], t2[9];
                const uint64_t u1 = __builtin_amdgcn_ballot_w64(a1 != 0.0f);  // use1 (alpha >= 1/255 > 0)
                const uint64_t u2 = __builtin_amdgcn_ballot_w64(a2 != 0.0f);
                auto step = [&](const float4& xc, float cb, float dx, float dy, float oG, float a, float rinv,
                                float* d) {
                    const float Tj = T * rinv;  // transmittance in front of the splat
                    const float w = a * Tj;
                    d[6] = w * g0;
                    d[7] = w * g1;
                    d[8] = w * g2;
                    const float gc = __builtin_fmaf(g2, cb, __builtin_fmaf(g1, xc.w, g0 * xc.z));  // g.c
                    const float wgc = w * gc;
                    // dL/dpower = alpha dL/dalpha = w (g.c) - alpha / (1 - alpha) (g.R),
                    // zero through a saturated alpha (o G > 0.99)
                    float dp = __builtin_fmaf(-(a * rinv), gR, wgc);
                    dp = oG <= kAlphaMax ? dp : 0.0f;
                    gR += wgc;  // exact no-op at a = 0
                    T = Tj;
                    // dL/dpower and its moments; with alpha = o G unclamped,
                    // dL/do = sum G dL/dalpha = (sum dL/dpower) / o, and the conic
                    // and mean gradients follow from the moments once per splat
                    d[5] = dp;
                    d[0] = dx * dp;    // dx dp
                    d[1] = dy * dp;    // dy dp
                    d[2] = dx * d[0];  // dx^2 dp
                    d[3] = dy * d[0];  // dx dy dp
                    d[4] = dy * d[1];  // dy^2 dp
                };
                step(xc1, cb1, dx1, dy1, oG1, a1, rinv1, t1);
                step(xc2, cb2, dx2, dy2, oG2, a2, rinv2, t2);
                if ((u1 | u2) != 0ull) {
                    const float r1 = transpose_row_sum9(t1[0], t1[1], t1[2], t1[3], t1[4], t1[5], t1[6], t1[7], t1[8],
                                                        lane_b0, lane_b1, lane_b2, lane_b3);
                    const float r2 = transpose_row_sum9(t2[0], t2[1], t2[2], t2[3], t2[4], t2[5], t2[6], t2[7], t2[8],
                                                        lane_b0, lane_b1, lane_b2, lane_b3);
                    if (store_lane) {
                        if (u1 != 0ull) store_base[k1 * store_stride] = r1;
                        if (u2 != 0ull) store_base[k2 * store_stride] = r2;
                    }
                    stored |= (u1 != 0ull ? 1u << k1 : 0u) | (u2 != 0ull ? 1u << k2 : 0u);
                }
            }
            if (lane == 0) s_wmask[wave] = stored;
            __syncthreads();
            // all 256 threads: splat slot k = tid % 32, one output group per
            // thread (tid / 32): the mean pair, dA, dB, dC, dopacity, r, g, b.
            // Only the partials of waves that wrote slot k in this batch count.
            //   d(u, v) = (A Sx + B Sy, B Sx + C Sy); dA = -Sxx / 2; dB = -Sxy; dC = -Syy / 2;
            //   do = S / o (S the sum of dL/dpower)
            {
                const int k = tid & (kBwdBatch - 1), grp = tid >> 5;
                if (k < cnt) {
                    uint32_t wm = 0u;
    #pragma unroll
                    for (int w = 0; w < 4; ++w) wm |= ((s_wmask[w] >> k) & 1u) << w;
                    if (wm != 0u) {
                        const uint32_t g = __float_as_uint(s_aux[off + k].y);
                        // term t of wave w sits in slots 4 w' .. 4 w' + 3, w' = w ^ part_swizzle(t) / 4
                        auto term_sum = [&](int t) {
                            const int flip = part_swizzle(t) >> 2;
                            float sum = 0.0f;
    #pragma unroll
                            for (int w = 0; w < 4; ++w) {
                                if ((wm >> w) & 1u) {
                                    const float4 q = reinterpret_cast<const float4*>(&s_part[k][t][0])[w ^ flip];
                                    sum += (q.x + q.y) + (q.z + q.w);
                                }
                            }
                            return sum;
                        };
                        if (grp == 0) {
                            const float4 co = s_conic[off + k];
                            const float Sx = term_sum(0), Sy = term_sum(1);
                            const float A = -2.0f * co.x, C = -2.0f * co.z;  // exact
                            atomic_add_nz(grad_mean2d + 2 * (size_t)g, A * Sx + co.y * Sy);
                            atomic_add_nz(grad_mean2d + 2 * (size_t)g + 1, co.y * Sx + C * Sy);
                        } else if (grp <= 3) {
                            const float scale = grp == 2 ? -1.0f : -0.5f;
                            atomic_add_nz(grad_conic_op + 4 * (size_t)g + (grp - 1), scale * term_sum(grp + 1));
                        } else if (grp == 4) {  // dL/do = (sum dL/dpower) / o
                            atomic_add_nz(grad_conic_op + 4 * (size_t)g + 3, term_sum(5) / s_conic[off + k].w);
                        } else {
                            atomic_add_nz(grad_rgb + 4 * (size_t)g + (grp - 5), term_sum(grp + 1));
                        }
                    }
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_composite_fwd(const gs_camera& cam, int n_views, const uint32_t* ranges,
                                const uint32_t* point_list, const float4* xy_depth,
                                const float4* conic_op, const float4* rgb, float3 bg,
                                float* image, float* final_T, uint32_t* n_contrib,
                                uint32_t* n_examined, const uint32_t* tile_order, float4* ckpt,
                                uint32_t capacity, const uint32_t* chunks, void* part, hipStream_t stream) {
    const int TX = tiles_x(cam), TYb = tiles_y(cam);
    const uint32_t n_tiles = (uint32_t)(TX * TYb * n_views);
    const uint32_t slots = (uint32_t)((capacity + (uint32_t)kChunk - 1u) / (uint32_t)kChunk);
    const uint32_t ckpt_slots = ckpt ? slots : 0u;
    if (chunks) {
        float4* const p4 = (float4*)part;
        uint32_t* const pl = (uint32_t*)(p4 + (size_t)(slots + n_tiles) * kChunk);
        hipLaunchKernelGGL(k_composite_fwd<true>, dim3(slots + n_tiles), dim3(256), 0, stream, cam.width, cam.height,
                           TX, TYb, (const uint32_t*)nullptr, point_list, xy_depth, conic_op, rgb, bg, image,
                           final_T, n_contrib, n_examined, (const uint32_t*)nullptr, ckpt, ckpt_slots, chunks,
                           n_tiles, slots, p4, pl);
        hipLaunchKernelGGL(k_composite_fwd_resolve, dim3(slots + n_tiles), dim3(256), 0, stream, cam.width,
                           cam.height, TX, TYb, point_list, xy_depth, conic_op, rgb, bg, image, final_T, n_contrib,
                           n_examined, ckpt, chunks, n_tiles, slots, (const float4*)p4, (const uint32_t*)pl);
    } else {
        hipLaunchKernelGGL(k_composite_fwd<false>, dim3(n_tiles), dim3(256), 0, stream, cam.width, cam.height,
                           TX, TYb, ranges, point_list, xy_depth, conic_op, rgb, bg, image, final_T, n_contrib,
                           n_examined, tile_order, ckpt, ckpt_slots, (const uint32_t*)nullptr, n_tiles, slots,
                           (float4*)nullptr, (uint32_t*)nullptr);
    }
    return hipGetLastError();
}

size_t composite_part_bytes(const gs_camera& cam, int n_views, uint32_t capacity) {
    const size_t slots = (capacity + (size_t)kChunk - 1) / kChunk;
    return (slots + (size_t)tiles_x(cam) * tiles_y(cam) * n_views) * kChunk * (sizeof(float4) + sizeof(uint32_t));
}

hipError_t launch_composite_bwd(const gs_camera& cam, int n_views, int n, const uint32_t* ranges,
                                const uint32_t* point_list, const float4* xy_depth,
                                const float4* conic_op, const float4* rgb, float3 bg,
                                const float* final_T, const uint32_t* n_contrib,
                                const float* dL_dimage, float2* grad_mean2d,
                                float4* grad_conic_op, float4* grad_rgb, const uint32_t* tile_order,
                                const uint32_t* chunks, uint32_t capacity, const float4* ckpt,
                                const float* image, hipStream_t stream) {
    if (n > 0)
        hipLaunchKernelGGL(k_zero_grads, dim3((n + 255) / 256), dim3(256), 0, stream, grad_mean2d,
                           grad_conic_op, grad_rgb, n);
    const int TX = tiles_x(cam), TYb = tiles_y(cam);
    const uint32_t n_tiles = (uint32_t)(TX * TYb * n_views);
    if (chunks) {
        // at most one chunk per non-empty list beyond its full ones
        const uint32_t slots = (uint32_t)((capacity + (uint32_t)kChunk - 1u) / (uint32_t)kChunk);
        hipLaunchKernelGGL(k_composite_bwd<true>, dim3(slots + n_tiles), dim3(256), 0, stream, cam.width,
                           cam.height, TX, TYb, ranges, point_list, xy_depth, conic_op, rgb, bg, final_T, n_contrib,
                           dL_dimage, (float*)grad_mean2d, (float*)grad_conic_op, (float*)grad_rgb, tile_order,
                           chunks, slots, n_tiles, ckpt, image);
    } else {
        hipLaunchKernelGGL(k_composite_bwd<false>, dim3(n_tiles), dim3(256), 0, stream, cam.width, cam.height,
                           TX, TYb, ranges, point_list, xy_depth, conic_op, rgb, bg, final_T, n_contrib, dL_dimage,
                           (float*)grad_mean2d, (float*)grad_conic_op, (float*)grad_rgb, tile_order,
                           (const uint32_t*)nullptr, 0u, n_tiles, (const float4*)nullptr, (const float*)nullptr);
    }
    return hipGetLastError();
}

}  // namespace gs
