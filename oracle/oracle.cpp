// Plain CPU oracle for the tile-based 3D Gaussian Splatting rasterizer.
//
// TEST INFRASTRUCTURE ONLY. This file is the slow, obviously-correct
// statement of what the GPU path computes. Only the tests, the smoke check
// and the CPU-baseline leg of the benchmark may load it. It shares no code,
// header, constant table or helper with the HIP library; the two meet only
// through plain arrays.
//
// Sources (the pages this follows; each function names its passage):
//   [rigel]  "rigel" GitHub README: sections "Projection", "Binning",
//            "Rasterization", "Backward", "Deliberate differences".
//   [zenn]   "3D Gaussian Splatting ビューワを作る": sections 2.1.1-2.1.2
//            (covariance, EWA), 2.2.3 (SH basis), 2.3.1 (conic), 2.3.3
//            (radius), 4.1 (prefix scan), 4.2 (duplicate), 4.3 (radix sort),
//            4.4 (tile ranges), 4.5 (tile render).
//   [learn-gs] "11 - Tiles: the actual 3DGS design": constants block,
//            prep_splats, tile_spans, build_tile_lists, "The kernel".
//
// Floating point: every preprocess quantity is computed in IEEE fp32 with
// the operation order written below, no contraction (build with
// -ffp-contract=off), so integer results (radius, tile span, keys) are
// decided in the same precision as the kernels. Compositing is templated on
// the real type: fp32 for parity, fp64 for finite-difference pins.
// Gradients are summed over pixels in double.
//
// Parity pins for every function live in tests/test_oracle_*.py.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

extern "C" {

// World-to-camera pinhole camera. p_cam = R p + t, R row-major; +z forward,
// image y down; campos is the camera centre in world space (-R^T t), given
// explicitly so every consumer uses the same bits.
typedef struct {
    float R[9];
    float t[3];
    float campos[3];
    float fx, fy, cx, cy;
    int32_t width, height;
} orc_camera;

}  // extern "C"

namespace {

// Constants. [learn-gs] constants block: DILATION 0.3, ALPHA_MIN 1/255,
// ALPHA_MAX 0.99, T_STOP 1e-4, Z_NEAR 0.05, TILE 16. [rigel] "Projection":
// x/z, y/z clamped to 1.3x the frustum half-width; 3 standard deviations.
// [zenn] 2.3.3: discriminant floor 0.1.
const int   TILE       = 16;
const float DILATION   = 0.3f;
const float Z_NEAR     = 0.05f;
const float FRUSTUM_CLAMP = 1.3f;
const float DISC_FLOOR = 0.1f;
const float SIGMA      = 3.0f;
const float ALPHA_MIN  = 1.0f / 255.0f;
const float ALPHA_MAX  = 0.99f;
const float T_STOP     = 1e-4f;

int tiles_x(const orc_camera* cam) { return (cam->width + TILE - 1) / TILE; }
int tiles_y(const orc_camera* cam) { return (cam->height + TILE - 1) / TILE; }

// Real spherical-harmonic basis, degrees 0..3, in the order and with the
// signs of [zenn] 2.2.3 (Sloan's polynomial forms). Each constant is rounded
// to fp32 from its closed form; each polynomial is evaluated left to right
// as written there.
struct ShConstants {
    float k[16];
    ShConstants() {
        const double pi = 3.14159265358979323846;
        k[0]  = (float)(0.5 / std::sqrt(pi));                   // 1/(2 sqrt(pi))
        k[1]  = (float)(-std::sqrt(3.0 / (4.0 * pi)));          // -sqrt(3/4pi) y
        k[2]  = (float)(std::sqrt(3.0 / (4.0 * pi)));           //  sqrt(3/4pi) z
        k[3]  = (float)(-std::sqrt(3.0 / (4.0 * pi)));          // -sqrt(3/4pi) x
        k[4]  = (float)(0.5 * std::sqrt(15.0 / pi));            //  xy
        k[5]  = (float)(-0.5 * std::sqrt(15.0 / pi));           //  yz
        k[6]  = (float)(0.25 * std::sqrt(5.0 / pi));            //  2z^2-x^2-y^2
        k[7]  = (float)(-0.5 * std::sqrt(15.0 / pi));           //  zx
        k[8]  = (float)(0.25 * std::sqrt(15.0 / pi));           //  x^2-y^2
        k[9]  = (float)(-0.25 * std::sqrt(35.0 / (2.0 * pi)));  //  (3x^2-y^2)y
        k[10] = (float)(0.5 * std::sqrt(105.0 / pi));           //  xyz
        k[11] = (float)(-0.25 * std::sqrt(21.0 / (2.0 * pi)));  //  (4z^2-x^2-y^2)y
        k[12] = (float)(0.25 * std::sqrt(7.0 / pi));            //  z(2z^2-3x^2-3y^2)
        k[13] = (float)(-0.25 * std::sqrt(21.0 / (2.0 * pi)));  //  x(4z^2-x^2-y^2)
        k[14] = (float)(0.25 * std::sqrt(105.0 / pi));          //  (x^2-y^2)z
        k[15] = (float)(-0.25 * std::sqrt(35.0 / (2.0 * pi)));  //  x(x^2-3y^2)
    }
};
const ShConstants SH;

void sh_basis(float x, float y, float z, float Y[16]) {
    const float xx = x * x, yy = y * y, zz = z * z;
    Y[0]  = SH.k[0];
    Y[1]  = SH.k[1] * y;
    Y[2]  = SH.k[2] * z;
    Y[3]  = SH.k[3] * x;
    Y[4]  = SH.k[4] * (x * y);
    Y[5]  = SH.k[5] * (y * z);
    Y[6]  = SH.k[6] * ((2.0f * zz - xx) - yy);
    Y[7]  = SH.k[7] * (z * x);
    Y[8]  = SH.k[8] * (xx - yy);
    Y[9]  = SH.k[9] * ((3.0f * xx - yy) * y);
    Y[10] = SH.k[10] * ((x * y) * z);
    Y[11] = SH.k[11] * (((4.0f * zz - xx) - yy) * y);
    Y[12] = SH.k[12] * (z * ((2.0f * zz - 3.0f * xx) - 3.0f * yy));
    Y[13] = SH.k[13] * (x * ((4.0f * zz - xx) - yy));
    Y[14] = SH.k[14] * ((xx - yy) * z);
    Y[15] = SH.k[15] * (x * (xx - 3.0f * yy));
}

// Tile span of a splat: the tiles its 2r square touches. [learn-gs]
// tile_spans: lo = clamp(floor((u - r)/16), 0, TX), hi = clamp(floor((u +
// r)/16) + 1, 0, TX), the same in y. Clamped in float, then converted.
struct Span { int x0, x1, y0, y1; };

Span tile_span(float u, float v, float r, int TX, int TY) {
    const float tile = (float)TILE;
    float x0 = std::floor((u - r) / tile);
    float x1 = std::floor((u + r) / tile) + 1.0f;
    float y0 = std::floor((v - r) / tile);
    float y1 = std::floor((v + r) / tile) + 1.0f;
    x0 = std::min(std::max(x0, 0.0f), (float)TX);
    x1 = std::min(std::max(x1, 0.0f), (float)TX);
    y0 = std::min(std::max(y0, 0.0f), (float)TY);
    y1 = std::min(std::max(y1, 0.0f), (float)TY);
    return Span{(int)x0, (int)x1, (int)y0, (int)y1};
}

inline uint32_t float_bits(float f) {
    uint32_t b;
    std::memcpy(&b, &f, 4);
    return b;
}

}  // namespace

extern "C" {

// Constants in a fixed order: tile, dilation, z_near, frustum clamp,
// discriminant floor, sigma, alpha_min, alpha_max, t_stop.
void orc_constants(float out[9]) {
    out[0] = (float)TILE; out[1] = DILATION; out[2] = Z_NEAR;
    out[3] = FRUSTUM_CLAMP; out[4] = DISC_FLOOR; out[5] = SIGMA;
    out[6] = ALPHA_MIN; out[7] = ALPHA_MAX; out[8] = T_STOP;
}

// The 16 SH basis values for a unit direction (exposed for the pins).
void orc_sh_basis(float x, float y, float z, float* out16) { sh_basis(x, y, z, out16); }

// Preprocess, one Gaussian at a time.
//   [rigel] "Projection": camera transform, explicit pinhole, EWA
//     Sigma_2d = J W Sigma W^T J^T + 0.3 I with x/z, y/z clamped to 1.3x the
//     half-width before J is built; conic; 3-sigma radius; radius 0 for
//     anything behind the near plane, degenerate or off-screen.
//   [zenn] 2.1.1: Sigma = R S S^T R^T; 2.1.2: J; 2.3.1: conic;
//     2.3.3: lambda_max with the 0.1 discriminant floor; 2.2.3: SH colour.
//   [learn-gs] prep_splats: z > Z_NEAR cull, u = fx x/z + cx, det > 0.
// Layouts: means/scales [3][n], quats [4][n] (w,x,y,z), opacity [n],
// sh [(d+1)^2][3][n] or NULL (then rgb_in [3][n]). Outputs per Gaussian:
// xy_depth (u, v, z, radius), conic_op (A, B, C, opacity), rgb (r, g, b, 0),
// tiles_touched. A culled Gaussian gets all-zero outputs.
// Returns 0, or -1 on an invalid argument.
int orc_preprocess(const orc_camera* cam, int32_t n, const float* means,
                   const float* scales, const float* quats, const float* opacity,
                   const float* sh, int32_t sh_degree, const float* rgb_in,
                   float* xy_depth, float* conic_op, float* rgb,
                   uint32_t* tiles_touched) {
    if (!cam || n < 0) return -1;
    if (sh && (sh_degree < 0 || sh_degree > 3)) return -1;
    const int TX = tiles_x(cam), TY = tiles_y(cam);
    const float* W = cam->R;  // the view rotation
    const int n_coef = sh ? (sh_degree + 1) * (sh_degree + 1) : 0;

    for (int g = 0; g < n; ++g) {
        float* o_xy = xy_depth + 4 * (size_t)g;
        float* o_co = conic_op + 4 * (size_t)g;
        float* o_rgb = rgb + 4 * (size_t)g;
        for (int k = 0; k < 4; ++k) { o_xy[k] = 0.0f; o_co[k] = 0.0f; o_rgb[k] = 0.0f; }
        tiles_touched[g] = 0;

        const float mx = means[g], my = means[n + g], mz = means[2 * n + g];

        // Camera space.
        const float px = ((W[0] * mx + W[1] * my) + W[2] * mz) + cam->t[0];
        const float py = ((W[3] * mx + W[4] * my) + W[5] * mz) + cam->t[1];
        const float pz = ((W[6] * mx + W[7] * my) + W[8] * mz) + cam->t[2];
        if (!(pz > Z_NEAR)) continue;  // also rejects NaN

        // Pinhole projection of the centre.
        const float u = (cam->fx * px) / pz + cam->cx;
        const float v = (cam->fy * py) / pz + cam->cy;
        if (!std::isfinite(u) || !std::isfinite(v)) continue;

        // Jacobian of the pinhole at the centre, x/z and y/z clamped.
        const float limx = FRUSTUM_CLAMP * ((0.5f * (float)cam->width) / cam->fx);
        const float limy = FRUSTUM_CLAMP * ((0.5f * (float)cam->height) / cam->fy);
        const float xj = std::min(limx, std::max(-limx, px / pz)) * pz;
        const float yj = std::min(limy, std::max(-limy, py / pz)) * pz;
        const float zz = pz * pz;
        const float J00 = cam->fx / pz;
        const float J02 = -(cam->fx * xj) / zz;
        const float J11 = cam->fy / pz;
        const float J12 = -(cam->fy * yj) / zz;

        // Rotation from the quaternion, normalised here.
        float qw = quats[g], qx = quats[n + g], qy = quats[2 * n + g], qz = quats[3 * n + g];
        const float qn = std::sqrt(((qw * qw + qx * qx) + qy * qy) + qz * qz);
        if (!(qn > 0.0f)) continue;
        qw = qw / qn; qx = qx / qn; qy = qy / qn; qz = qz / qn;
        float Rq[3][3];
        Rq[0][0] = 1.0f - 2.0f * (qy * qy + qz * qz);
        Rq[0][1] = 2.0f * (qx * qy - qw * qz);
        Rq[0][2] = 2.0f * (qx * qz + qw * qy);
        Rq[1][0] = 2.0f * (qx * qy + qw * qz);
        Rq[1][1] = 1.0f - 2.0f * (qx * qx + qz * qz);
        Rq[1][2] = 2.0f * (qy * qz - qw * qx);
        Rq[2][0] = 2.0f * (qx * qz - qw * qy);
        Rq[2][1] = 2.0f * (qy * qz + qw * qx);
        Rq[2][2] = 1.0f - 2.0f * (qx * qx + qy * qy);

        // Sigma = (R S)(R S)^T.
        const float s[3] = {scales[g], scales[n + g], scales[2 * n + g]};
        float M[3][3];
        for (int i = 0; i < 3; ++i)
            for (int j = 0; j < 3; ++j) M[i][j] = Rq[i][j] * s[j];
        float Sig[3][3];
        for (int i = 0; i < 3; ++i)
            for (int j = 0; j < 3; ++j)
                Sig[i][j] = (M[i][0] * M[j][0] + M[i][1] * M[j][1]) + M[i][2] * M[j][2];

        // T = J W (J's structural zeros skipped), U = T Sigma, Sigma_2d = U T^T.
        float T[2][3];
        for (int j = 0; j < 3; ++j) {
            T[0][j] = J00 * W[0 * 3 + j] + J02 * W[2 * 3 + j];
            T[1][j] = J11 * W[1 * 3 + j] + J12 * W[2 * 3 + j];
        }
        float U[2][3];
        for (int i = 0; i < 2; ++i)
            for (int j = 0; j < 3; ++j)
                U[i][j] = (T[i][0] * Sig[0][j] + T[i][1] * Sig[1][j]) + T[i][2] * Sig[2][j];
        const float a = ((U[0][0] * T[0][0] + U[0][1] * T[0][1]) + U[0][2] * T[0][2]) + DILATION;
        const float b = (U[0][0] * T[1][0] + U[0][1] * T[1][1]) + U[0][2] * T[1][2];
        const float c = ((U[1][0] * T[1][0] + U[1][1] * T[1][1]) + U[1][2] * T[1][2]) + DILATION;

        // Conic and degenerate cull (non-finite covariances are culled too).
        if (!std::isfinite(a) || !std::isfinite(b) || !std::isfinite(c)) continue;
        const float det = a * c - b * b;
        if (!(det > 0.0f) || !std::isfinite(det)) continue;
        const float cA = c / det, cB = -b / det, cC = a / det;

        // Bounding radius: 3 sqrt(lambda_max), discriminant floored at 0.1.
        const float mid = 0.5f * (a + c);
        const float lam = mid + std::sqrt(std::max(mid * mid - det, DISC_FLOOR));
        const float r = std::ceil(SIGMA * std::sqrt(lam));
        if (!std::isfinite(r)) continue;

        // Tile span; nothing on screen means culled.
        const Span sp = tile_span(u, v, r, TX, TY);
        const int count = (sp.x1 - sp.x0) * (sp.y1 - sp.y0);
        if (count <= 0) continue;

        // Colour: SH evaluated at the unit direction from the camera centre.
        float col[3];
        if (sh) {
            float dx = mx - cam->campos[0], dy = my - cam->campos[1], dz = mz - cam->campos[2];
            const float dn = std::sqrt((dx * dx + dy * dy) + dz * dz);
            dx = dx / dn; dy = dy / dn; dz = dz / dn;
            float Y[16];
            sh_basis(dx, dy, dz, Y);
            for (int ch = 0; ch < 3; ++ch) {
                float acc = sh[(size_t)(0 * 3 + ch) * n + g] * Y[0];
                for (int k = 1; k < n_coef; ++k) acc = acc + sh[(size_t)(k * 3 + ch) * n + g] * Y[k];
                col[ch] = acc;
            }
        } else {
            for (int ch = 0; ch < 3; ++ch) col[ch] = rgb_in[(size_t)ch * n + g];
        }
        // A Gaussian whose opacity or colour is not finite is culled as well.
        if (!std::isfinite(opacity[g]) || !std::isfinite(col[0]) || !std::isfinite(col[1]) ||
            !std::isfinite(col[2])) continue;

        o_xy[0] = u; o_xy[1] = v; o_xy[2] = pz; o_xy[3] = r;
        o_co[0] = cA; o_co[1] = cB; o_co[2] = cC; o_co[3] = opacity[g];
        o_rgb[0] = col[0]; o_rgb[1] = col[1]; o_rgb[2] = col[2];
        tiles_touched[g] = (uint32_t)count;
    }
    return 0;
}

// Tile span of one splat (exposed for the pins): out = x0, x1, y0, y1.
void orc_tile_span(float u, float v, float r, int32_t TX, int32_t TY, int32_t* out) {
    const Span sp = tile_span(u, v, r, TX, TY);
    out[0] = sp.x0; out[1] = sp.x1; out[2] = sp.y0; out[3] = sp.y1;
}

// Exclusive prefix sum of the per-Gaussian tile counts: Gaussian g owns the
// entries [offsets[g], offsets[g] + counts[g]). Returns the total.
//   [zenn] 4.1.1 (exclusive scan as slice starts), [rigel] "Binning"
//   (a scan gives every Gaussian a private slice).
uint64_t orc_exclusive_scan(const uint32_t* counts, int64_t n, uint64_t* offsets) {
    uint64_t total = 0;
    for (int64_t i = 0; i < n; ++i) { offsets[i] = total; total += counts[i]; }
    return total;
}

// Duplication: each Gaussian writes one (key, value) pair per covered tile
// into its own slice, tiles in span order (ty outer, tx inner);
// key = (tile_id << 32) | float_bits(depth), value = Gaussian index.
//   [rigel] "Binning" (the key), [zenn] 4.2 (pair_key / pair_value, written
//   at offsets), [learn-gs] build_tile_lists (tile_id = ty*TX + tx).
// Returns 0, or -2 if a Gaussian's span disagrees with its count.
int orc_duplicate(const orc_camera* cam, int32_t n, const float* xy_depth,
                  const uint32_t* tiles_touched, const uint64_t* offsets,
                  uint64_t* keys, uint32_t* values) {
    const int TX = tiles_x(cam), TY = tiles_y(cam);
    for (int g = 0; g < n; ++g) {
        if (tiles_touched[g] == 0) continue;
        const float* rec = xy_depth + 4 * (size_t)g;
        const Span sp = tile_span(rec[0], rec[1], rec[3], TX, TY);
        if ((uint32_t)((sp.x1 - sp.x0) * (sp.y1 - sp.y0)) != tiles_touched[g]) return -2;
        const uint64_t depth_bits = float_bits(rec[2]);
        uint64_t k = offsets[g];
        for (int ty = sp.y0; ty < sp.y1; ++ty)
            for (int tx = sp.x0; tx < sp.x1; ++tx) {
                keys[k] = ((uint64_t)(ty * TX + tx) << 32) | depth_bits;
                values[k] = (uint32_t)g;
                ++k;
            }
    }
    return 0;
}

// One stable sort of the pairs by key, ascending: ties keep their input
// order. [rigel] "Binning" (one sort yields tile-major, front-to-back
// order), [zenn] 4.3.
void orc_sort_pairs(uint64_t* keys, uint32_t* values, int64_t n) {
    std::vector<std::pair<uint64_t, uint32_t>> kv((size_t)n);
    for (int64_t i = 0; i < n; ++i) kv[i] = {keys[i], values[i]};
    std::stable_sort(kv.begin(), kv.end(),
                     [](const std::pair<uint64_t, uint32_t>& x,
                        const std::pair<uint64_t, uint32_t>& y) { return x.first < y.first; });
    for (int64_t i = 0; i < n; ++i) { keys[i] = kv[i].first; values[i] = kv[i].second; }
}

// Binning end to end: scan, duplicate, sort. Returns the entry count E (also
// when capacity < E, in which case nothing is written), -1 on an invalid
// argument, -2 if a count disagrees with its span.
int64_t orc_bin(const orc_camera* cam, int32_t n, const float* xy_depth,
                const uint32_t* tiles_touched, uint64_t* keys, uint32_t* point_list,
                int64_t capacity) {
    if (!cam || n < 0) return -1;
    std::vector<uint64_t> offsets((size_t)n);
    const uint64_t total = orc_exclusive_scan(tiles_touched, n, offsets.data());
    if ((int64_t)total > capacity) return (int64_t)total;
    if (orc_duplicate(cam, n, xy_depth, tiles_touched, offsets.data(), keys, point_list) != 0) return -2;
    orc_sort_pairs(keys, point_list, (int64_t)total);
    return (int64_t)total;
}

// Tile ranges over the sorted keys: ranges[t] = [start, end) of tile t's
// run; an absent tile gets (0, 0).  [zenn] 4.4.1-4.4.2, [rigel] "Binning".
void orc_tile_ranges(const orc_camera* cam, const uint64_t* keys, int64_t n_entries,
                     uint32_t* ranges) {
    const int n_tiles = tiles_x(cam) * tiles_y(cam);
    for (int t = 0; t < n_tiles; ++t) { ranges[2 * t] = 0; ranges[2 * t + 1] = 0; }
    for (int64_t i = 0; i < n_entries; ++i) {
        const uint32_t t = (uint32_t)(keys[i] >> 32);
        if (i == 0 || (uint32_t)(keys[i - 1] >> 32) != t) ranges[2 * t] = (uint32_t)i;
        if (i == n_entries - 1 || (uint32_t)(keys[i + 1] >> 32) != t) ranges[2 * t + 1] = (uint32_t)(i + 1);
    }
}

}  // extern "C"

namespace {

// The exponential of the compositing step. The pages leave its precision
// open; in fp32 it is the correctly rounded value (evaluated in double and
// rounded once), so the alpha-floor and stop decisions are taken on an
// exactly defined number. In fp64 it is the double exponential.
inline float exp_rn(float x) { return (float)std::exp((double)x); }
inline double exp_rn(double x) { return std::exp(x); }

// Forward compositing of one image, front to back per pixel over its tile's
// depth-sorted list.
//   [rigel] "Rasterization": power = -0.5 (A dx^2 + C dy^2) - B dx dy,
//     alpha = min(0.99, opacity exp(power)), C += colour alpha T,
//     T *= 1 - alpha, stop once T < 1e-4.
//   [learn-gs] constants: alpha below 1/255 does not pass (skipped).
//   [zenn] 4.5.5: accumulate, update T, then test the stop threshold.
//   [rigel] "Backward": image = sum c_i a_i T_i + T_final bg.
// Pixel (x, y) is sampled at its integer coordinates; dx = x - u.
// n_contrib = 1 + list position of the last contributing splat (0 if none);
// n_examined = splats evaluated before stopping (diagnostic).
template <typename F>
void composite_fwd(const orc_camera* cam, const uint32_t* ranges, const uint32_t* point_list,
                   const F* xy_depth, const F* conic_op, const F* rgb, const F* bg,
                   F* image, F* final_T, uint32_t* n_contrib, uint32_t* n_examined) {
    const int Wd = cam->width, Hd = cam->height, TX = tiles_x(cam);
    const F alpha_min = (F)ALPHA_MIN, alpha_max = (F)ALPHA_MAX, t_stop = (F)T_STOP;
    for (int y = 0; y < Hd; ++y) {
        for (int x = 0; x < Wd; ++x) {
            const int tile = (y / TILE) * TX + (x / TILE);
            const uint32_t start = ranges[2 * tile], end = ranges[2 * tile + 1];
            F T = 1, C[3] = {0, 0, 0};
            uint32_t last = 0, examined = 0;
            for (uint32_t j = start; j < end; ++j) {
                const uint32_t g = point_list[j];
                const F* co = conic_op + 4 * (size_t)g;
                const F dx = (F)x - xy_depth[4 * (size_t)g + 0];
                const F dy = (F)y - xy_depth[4 * (size_t)g + 1];
                const F power = (F)(-0.5) * ((co[0] * dx) * dx + (co[2] * dy) * dy) - (co[1] * dx) * dy;
                const F G = exp_rn(power);
                const F alpha = std::min(alpha_max, co[3] * G);
                examined = j - start + 1;
                if (alpha < alpha_min) continue;
                const F w = alpha * T;
                for (int ch = 0; ch < 3; ++ch) C[ch] = C[ch] + rgb[4 * (size_t)g + ch] * w;
                T = T * ((F)1 - alpha);
                last = j - start + 1;
                if (T < t_stop) break;
            }
            const size_t p = (size_t)y * Wd + x;
            for (int ch = 0; ch < 3; ++ch) image[(size_t)ch * Hd * Wd + p] = C[ch] + T * bg[ch];
            final_T[p] = T;
            n_contrib[p] = last;
            if (n_examined) n_examined[p] = examined;
        }
    }
}

// Backward of composite_fwd: walk each pixel's list back to front from
// n_contrib - 1, undoing T_j = T_{j+1} / (1 - a_j) from final_T and carrying
// the colour behind the current splat (starting from the background).
//   [rigel] "Backward": suffix accumulation, T recovery, n_contrib skip;
//     "Deliberate differences": zero gradient through a saturated alpha.
//   [learn-gs] "The next live problem": the tile walk in reverse,
//     reconstructing each T_i from the end state.
// Per splat j with colour c, alpha a (unclamped a_raw = o G), and upstream
// pixel gradient g:  dL/dc = a T_j g;  dL/da = T_j sum_ch g_ch (c_ch - B_ch),
// where B is the colour behind j; when a_raw <= 0.99, dL/do = G dL/da and
// dL/dpower = a dL/da feed dA, dB, dC, du, dv. Summed over pixels in double.
// Outputs: grad_mean2d [n][2], grad_conic_op [n][4] (dA, dB, dC, dopacity),
// grad_rgb [n][4] (last slot 0). They are overwritten.
template <typename F>
void composite_bwd(const orc_camera* cam, int32_t n, const uint32_t* ranges,
                   const uint32_t* point_list, const F* xy_depth, const F* conic_op,
                   const F* rgb, const F* bg, const F* final_T, const uint32_t* n_contrib,
                   const F* dL_dimage, double* grad_mean2d, double* grad_conic_op,
                   double* grad_rgb) {
    const int Wd = cam->width, Hd = cam->height, TX = tiles_x(cam);
    const F alpha_min = (F)ALPHA_MIN, alpha_max = (F)ALPHA_MAX;
    std::fill(grad_mean2d, grad_mean2d + 2 * (size_t)n, 0.0);
    std::fill(grad_conic_op, grad_conic_op + 4 * (size_t)n, 0.0);
    std::fill(grad_rgb, grad_rgb + 4 * (size_t)n, 0.0);
    for (int y = 0; y < Hd; ++y) {
        for (int x = 0; x < Wd; ++x) {
            const int tile = (y / TILE) * TX + (x / TILE);
            const uint32_t start = ranges[2 * tile];
            const size_t p = (size_t)y * Wd + x;
            F gpix[3], B[3];
            for (int ch = 0; ch < 3; ++ch) { gpix[ch] = dL_dimage[(size_t)ch * Hd * Wd + p]; B[ch] = bg[ch]; }
            F T = final_T[p];
            for (int64_t jj = (int64_t)n_contrib[p] - 1; jj >= 0; --jj) {
                const uint32_t g = point_list[start + (uint32_t)jj];
                const F* co = conic_op + 4 * (size_t)g;
                const F* c = rgb + 4 * (size_t)g;
                const F dx = (F)x - xy_depth[4 * (size_t)g + 0];
                const F dy = (F)y - xy_depth[4 * (size_t)g + 1];
                const F power = (F)(-0.5) * ((co[0] * dx) * dx + (co[2] * dy) * dy) - (co[1] * dx) * dy;
                const F G = exp_rn(power);
                const F a_raw = co[3] * G;
                const F a = std::min(alpha_max, a_raw);
                if (a < alpha_min) continue;
                const F Tj = T / ((F)1 - a);
                F dL_da = 0;
                for (int ch = 0; ch < 3; ++ch) {
                    grad_rgb[4 * (size_t)g + ch] += (double)(a * Tj * gpix[ch]);
                    dL_da = dL_da + gpix[ch] * (c[ch] - B[ch]);
                }
                dL_da = dL_da * Tj;
                for (int ch = 0; ch < 3; ++ch) B[ch] = a * c[ch] + ((F)1 - a) * B[ch];
                T = Tj;
                if (a_raw > alpha_max) continue;  // saturated: no gradient to o, conic, mean
                const F dp = a * dL_da;
                grad_conic_op[4 * (size_t)g + 3] += (double)(G * dL_da);
                grad_conic_op[4 * (size_t)g + 0] += (double)((F)(-0.5) * dx * dx * dp);
                grad_conic_op[4 * (size_t)g + 1] += (double)(-dx * dy * dp);
                grad_conic_op[4 * (size_t)g + 2] += (double)((F)(-0.5) * dy * dy * dp);
                grad_mean2d[2 * (size_t)g + 0] += (double)((co[0] * dx + co[1] * dy) * dp);
                grad_mean2d[2 * (size_t)g + 1] += (double)((co[1] * dx + co[2] * dy) * dp);
            }
        }
    }
}

}  // namespace

extern "C" {

void orc_composite_fwd_f32(const orc_camera* cam, const uint32_t* ranges, const uint32_t* point_list,
                           const float* xy_depth, const float* conic_op, const float* rgb,
                           const float* bg, float* image, float* final_T, uint32_t* n_contrib,
                           uint32_t* n_examined) {
    composite_fwd<float>(cam, ranges, point_list, xy_depth, conic_op, rgb, bg, image, final_T,
                         n_contrib, n_examined);
}

void orc_composite_fwd_f64(const orc_camera* cam, const uint32_t* ranges, const uint32_t* point_list,
                           const double* xy_depth, const double* conic_op, const double* rgb,
                           const double* bg, double* image, double* final_T, uint32_t* n_contrib,
                           uint32_t* n_examined) {
    composite_fwd<double>(cam, ranges, point_list, xy_depth, conic_op, rgb, bg, image, final_T,
                          n_contrib, n_examined);
}

void orc_composite_bwd_f32(const orc_camera* cam, int32_t n, const uint32_t* ranges,
                           const uint32_t* point_list, const float* xy_depth, const float* conic_op,
                           const float* rgb, const float* bg, const float* final_T,
                           const uint32_t* n_contrib, const float* dL_dimage, double* grad_mean2d,
                           double* grad_conic_op, double* grad_rgb) {
    composite_bwd<float>(cam, n, ranges, point_list, xy_depth, conic_op, rgb, bg, final_T,
                         n_contrib, dL_dimage, grad_mean2d, grad_conic_op, grad_rgb);
}

void orc_composite_bwd_f64(const orc_camera* cam, int32_t n, const uint32_t* ranges,
                           const uint32_t* point_list, const double* xy_depth, const double* conic_op,
                           const double* rgb, const double* bg, const double* final_T,
                           const uint32_t* n_contrib, const double* dL_dimage, double* grad_mean2d,
                           double* grad_conic_op, double* grad_rgb) {
    composite_bwd<double>(cam, n, ranges, point_list, xy_depth, conic_op, rgb, bg, final_T,
                          n_contrib, dL_dimage, grad_mean2d, grad_conic_op, grad_rgb);
}

}  // extern "C"
