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

#include <omp.h>

// Threads used by the preprocess and the compositing (orc_set_threads).
// At 1, the default, every loop runs in the order written below. Above 1
// the preprocess (per Gaussian) and the forward (per pixel row) split
// independent iterations over threads, so their outputs are identical; the
// backward gives each thread its own partial gradients over a block of
// rows and sums them in thread order, so its sums differ from the
// single-threaded ones by double rounding only. Used to time the oracle on
// all host cores; the pins run single-threaded.
static int g_threads = 1;

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

template <typename F>
void sh_basis(F x, F y, F z, F Y[16]) {
    const F xx = x * x, yy = y * y, zz = z * z;
    const F* k = nullptr;
    F kk[16];
    for (int i = 0; i < 16; ++i) kk[i] = (F)SH.k[i];
    k = kk;
    Y[0]  = k[0];
    Y[1]  = k[1] * y;
    Y[2]  = k[2] * z;
    Y[3]  = k[3] * x;
    Y[4]  = k[4] * (x * y);
    Y[5]  = k[5] * (y * z);
    Y[6]  = k[6] * (((F)2 * zz - xx) - yy);
    Y[7]  = k[7] * (z * x);
    Y[8]  = k[8] * (xx - yy);
    Y[9]  = k[9] * (((F)3 * xx - yy) * y);
    Y[10] = k[10] * ((x * y) * z);
    Y[11] = k[11] * ((((F)4 * zz - xx) - yy) * y);
    Y[12] = k[12] * (z * (((F)2 * zz - (F)3 * xx) - (F)3 * yy));
    Y[13] = k[13] * (x * (((F)4 * zz - xx) - yy));
    Y[14] = k[14] * ((xx - yy) * z);
    Y[15] = k[15] * (x * (xx - (F)3 * yy));
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

// Ellipse tile test ([zenn] 2.3.4: of the tiles in the span rectangle, keep
// those the splat's ellipse may overlap). The page does not give the test;
// the reading taken: the ellipse is the region where the splat can reach
// alpha >= 1/255, Q(d) = A dx^2 + 2B dx dy + C dy^2 <= 2 ln(255 o) <= 2 ln 255,
// taken with the opacity-independent threshold 11.1 (> 2 ln 255 = 11.0825)
// raised by a bound on the compositing's fp32 rounding of Q, so a dropped
// tile holds no pixel the splat changes and the image is unchanged. Per
// row of tiles, the kept tiles are those whose pixel centres meet the
// x-extent [L, R] of the ellipse's slice over the row's pixel-centre
// y-range; L and R are the slice edges at the dy of the ellipse's leftmost
// and rightmost points, clamped into the row (the edges are convex and
// concave in dy), widened by a slack. Every step is + - * / sqrt floor ceil
// fminf fmaxf in float32 in the order written, so the kernels can take the
// identical decision. A conic that is not positive definite, or anything
// not finite, keeps the whole span.
struct EllipseRows {
    bool full;  // keep every tile of the span
    float u, v, A, B, C, det, hx, hy, ydr, slack, thr;
};

EllipseRows ellipse_rows(float u, float v, float A, float B, float C, const Span& sp) {
    EllipseRows e;
    e.u = u; e.v = v; e.A = A; e.B = B; e.C = C;
    e.det = A * C - B * B;
    e.full = !(e.det > 0.0f && A > 0.0f && C > 0.0f);
    // farthest pixel centre of the span from the centre, per axis
    const float ex = fmaxf(fabsf(16.0f * (float)sp.x0 - u), fabsf(16.0f * (float)sp.x1 - 1.0f - u));
    const float ey = fmaxf(fabsf(16.0f * (float)sp.y0 - v), fabsf(16.0f * (float)sp.y1 - 1.0f - v));
    const float bound = 64.0f * 5.96e-8f * ((fabsf(A) + fabsf(C)) + 2.0f * fabsf(B)) * (ex * ex + ey * ey);
    e.thr = 11.1f + bound;
    if (e.full) return e;
    e.hy = std::sqrt((e.thr * A) / e.det);
    e.hx = std::sqrt((e.thr * C) / e.det);
    e.ydr = -(B * e.hx) / C;
    e.slack = 0.01f + 1e-4f * (e.hx + e.hy);
    if (!std::isfinite(e.hx) || !std::isfinite(e.hy) || !std::isfinite(e.ydr) || !std::isfinite(e.slack))
        e.full = true;
    return e;
}

// Kept tiles [lo, hi) of row ty (within the span's [x0, x1)); lo >= hi: none.
void ellipse_row_range(const EllipseRows& e, const Span& sp, int ty, int* lo_out, int* hi_out) {
    if (e.full) { *lo_out = sp.x0; *hi_out = sp.x1; return; }
    const float ylo = 16.0f * (float)ty - e.v;
    const float lo = fmaxf(ylo, -e.hy), hi = fminf(ylo + 15.0f, e.hy);
    if (lo > hi + e.slack) { *lo_out = sp.x0; *hi_out = sp.x0; return; }
    const float yr = fminf(fmaxf(e.ydr, lo), hi);
    const float yl = fminf(fmaxf(-e.ydr, lo), hi);
    const float thrA = e.thr * e.A;
    const float R = (-(e.B * yr) + std::sqrt(fmaxf(0.0f, thrA - (e.det * yr) * yr))) / e.A + e.slack;
    const float L = (-(e.B * yl) - std::sqrt(fmaxf(0.0f, thrA - (e.det * yl) * yl))) / e.A - e.slack;
    // tile tx has pixel centres [16 tx - u, 16 tx + 15 - u]
    const float tlo = fmaxf(std::ceil(((L + e.u) - 15.0f) / 16.0f), (float)sp.x0);
    const float thi = fminf(std::floor((R + e.u) / 16.0f) + 1.0f, (float)sp.x1);
    if (!(tlo < thi)) { *lo_out = sp.x0; *hi_out = sp.x0; return; }
    *lo_out = (int)tlo;
    *hi_out = (int)thi;
}

inline uint32_t float_bits(float f) {
    uint32_t b;
    std::memcpy(&b, &f, 4);
    return b;
}

// Projection of one Gaussian: every continuous quantity of the preprocess,
// in the real type F with the operation order below. F = float is the
// preprocess itself (bit-exact reference for the kernels); F = double is the
// same function widened, used only as the function that finite differences
// of the projection backward are taken of.
//   [rigel] "Projection": camera transform, explicit pinhole, EWA
//     Sigma_2d = J W Sigma W^T J^T + 0.3 I with x/z, y/z clamped to 1.3x the
//     half-width before J is built; conic; 3-sigma radius; radius 0 for
//     anything behind the near plane, degenerate or off-screen.
//   [zenn] 2.1.1: Sigma = R S S^T R^T; 2.1.2: J; 2.3.1: conic;
//     2.3.3: lambda_max with the 0.1 discriminant floor; 2.2.3: SH colour.
//   [learn-gs] prep_splats: z > Z_NEAR cull, u = fx x/z + cx, det > 0.
// sh_g: this Gaussian's coefficients [k][channel] (n_coef of them), or
// NULL, then rgb_g holds its colour. Returns false when the Gaussian is
// culled before the tile span is known (near plane, non-finite, zero
// quaternion, det <= 0); the span cull is the caller's.
template <typename F>
struct Projected {
    F u, v, z, r;
    F a, b, c;     // Sigma_2d with the dilation
    F A, B, C;     // conic
    F col[3];
    bool clamp_x, clamp_y;  // was x/z (y/z) clamped when J was built
};

template <typename F>
bool project_gaussian(const orc_camera* cam, const F m[3], const F s3[3], const F q[4],
                      const F* sh_g, int n_coef, const F* rgb_g, Projected<F>* out) {
    const F W[9] = {(F)cam->R[0], (F)cam->R[1], (F)cam->R[2], (F)cam->R[3], (F)cam->R[4],
                    (F)cam->R[5], (F)cam->R[6], (F)cam->R[7], (F)cam->R[8]};
    const F fx = (F)cam->fx, fy = (F)cam->fy;
    const F mx = m[0], my = m[1], mz = m[2];

    // Camera space.
    const F px = ((W[0] * mx + W[1] * my) + W[2] * mz) + (F)cam->t[0];
    const F py = ((W[3] * mx + W[4] * my) + W[5] * mz) + (F)cam->t[1];
    const F pz = ((W[6] * mx + W[7] * my) + W[8] * mz) + (F)cam->t[2];
    if (!(pz > (F)Z_NEAR)) return false;  // also rejects NaN

    // Pinhole projection of the centre.
    const F u = (fx * px) / pz + (F)cam->cx;
    const F v = (fy * py) / pz + (F)cam->cy;
    if (!std::isfinite(u) || !std::isfinite(v)) return false;

    // Jacobian of the pinhole at the centre, x/z and y/z clamped.
    const F limx = (F)FRUSTUM_CLAMP * (((F)0.5 * (F)cam->width) / fx);
    const F limy = (F)FRUSTUM_CLAMP * (((F)0.5 * (F)cam->height) / fy);
    const F tx = px / pz, ty = py / pz;
    const F xj = std::min(limx, std::max(-limx, tx)) * pz;
    const F yj = std::min(limy, std::max(-limy, ty)) * pz;
    const F zz = pz * pz;
    const F J00 = fx / pz;
    const F J02 = -(fx * xj) / zz;
    const F J11 = fy / pz;
    const F J12 = -(fy * yj) / zz;

    // Rotation from the quaternion, normalised here.
    F qw = q[0], qx = q[1], qy = q[2], qz = q[3];
    const F qn = std::sqrt(((qw * qw + qx * qx) + qy * qy) + qz * qz);
    if (!(qn > (F)0)) return false;
    qw = qw / qn; qx = qx / qn; qy = qy / qn; qz = qz / qn;
    F Rq[3][3];
    Rq[0][0] = (F)1 - (F)2 * (qy * qy + qz * qz);
    Rq[0][1] = (F)2 * (qx * qy - qw * qz);
    Rq[0][2] = (F)2 * (qx * qz + qw * qy);
    Rq[1][0] = (F)2 * (qx * qy + qw * qz);
    Rq[1][1] = (F)1 - (F)2 * (qx * qx + qz * qz);
    Rq[1][2] = (F)2 * (qy * qz - qw * qx);
    Rq[2][0] = (F)2 * (qx * qz - qw * qy);
    Rq[2][1] = (F)2 * (qy * qz + qw * qx);
    Rq[2][2] = (F)1 - (F)2 * (qx * qx + qy * qy);

    // Sigma = (R S)(R S)^T.
    F M[3][3];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) M[i][j] = Rq[i][j] * s3[j];
    F Sig[3][3];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            Sig[i][j] = (M[i][0] * M[j][0] + M[i][1] * M[j][1]) + M[i][2] * M[j][2];

    // T = J W (J's structural zeros skipped), U = T Sigma, Sigma_2d = U T^T.
    F T[2][3];
    for (int j = 0; j < 3; ++j) {
        T[0][j] = J00 * W[0 * 3 + j] + J02 * W[2 * 3 + j];
        T[1][j] = J11 * W[1 * 3 + j] + J12 * W[2 * 3 + j];
    }
    F U[2][3];
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 3; ++j)
            U[i][j] = (T[i][0] * Sig[0][j] + T[i][1] * Sig[1][j]) + T[i][2] * Sig[2][j];
    const F a = ((U[0][0] * T[0][0] + U[0][1] * T[0][1]) + U[0][2] * T[0][2]) + (F)DILATION;
    const F b = (U[0][0] * T[1][0] + U[0][1] * T[1][1]) + U[0][2] * T[1][2];
    const F c = ((U[1][0] * T[1][0] + U[1][1] * T[1][1]) + U[1][2] * T[1][2]) + (F)DILATION;

    // Conic and degenerate cull (non-finite covariances are culled too).
    if (!std::isfinite(a) || !std::isfinite(b) || !std::isfinite(c)) return false;
    const F det = a * c - b * b;
    if (!(det > (F)0) || !std::isfinite(det)) return false;

    // Bounding radius: 3 sqrt(lambda_max), discriminant floored at 0.1.
    const F mid = (F)0.5 * (a + c);
    const F lam = mid + std::sqrt(std::max(mid * mid - det, (F)DISC_FLOOR));
    const F r = std::ceil((F)SIGMA * std::sqrt(lam));
    if (!std::isfinite(r)) return false;

    // Colour: SH evaluated at the unit direction from the camera centre.
    if (sh_g) {
        F dx = mx - (F)cam->campos[0], dy = my - (F)cam->campos[1], dz = mz - (F)cam->campos[2];
        const F dn = std::sqrt((dx * dx + dy * dy) + dz * dz);
        dx = dx / dn; dy = dy / dn; dz = dz / dn;
        F Y[16];
        sh_basis(dx, dy, dz, Y);
        for (int ch = 0; ch < 3; ++ch) {
            F acc = sh_g[0 * 3 + ch] * Y[0];
            for (int k = 1; k < n_coef; ++k) acc = acc + sh_g[k * 3 + ch] * Y[k];
            out->col[ch] = acc;
        }
    } else {
        for (int ch = 0; ch < 3; ++ch) out->col[ch] = rgb_g[ch];
    }
    out->u = u; out->v = v; out->z = pz; out->r = r;
    out->a = a; out->b = b; out->c = c;
    out->A = c / det; out->B = -b / det; out->C = a / det;
    out->clamp_x = !(tx >= -limx && tx <= limx);
    out->clamp_y = !(ty >= -limy && ty <= limy);
    return true;
}

// Gathers Gaussian g's inputs from the structure-of-arrays layout.
template <typename F, typename In>
void gather_gaussian(int32_t n, int g, const In* means, const In* scales, const In* quats,
                     const In* sh, int n_coef, const In* rgb_in, F m[3], F s3[3], F q[4],
                     F sh_g[48], F rgb_g[3]) {
    for (int i = 0; i < 3; ++i) {
        m[i] = (F)means[(size_t)i * n + g];
        s3[i] = (F)scales[(size_t)i * n + g];
    }
    for (int i = 0; i < 4; ++i) q[i] = (F)quats[(size_t)i * n + g];
    for (int k = 0; k < n_coef; ++k)
        for (int ch = 0; ch < 3; ++ch) sh_g[k * 3 + ch] = (F)sh[(size_t)(k * 3 + ch) * n + g];
    if (rgb_in)
        for (int ch = 0; ch < 3; ++ch) rgb_g[ch] = (F)rgb_in[(size_t)ch * n + g];
}

// Gradient of the SH basis polynomials with respect to the direction
// components (x, y, z), differentiated term by term from the forms in
// sh_basis ([zenn] 2.2.3). dY[k][0..2] = dY_k/dx, dY_k/dy, dY_k/dz.
void sh_basis_grad(double x, double y, double z, double dY[16][3]) {
    double k[16];
    for (int i = 0; i < 16; ++i) k[i] = (double)SH.k[i];
    const double xx = x * x, yy = y * y, zz = z * z;
    const double g[16][3] = {
        {0, 0, 0},
        {0, k[1], 0},
        {0, 0, k[2]},
        {k[3], 0, 0},
        {k[4] * y, k[4] * x, 0},
        {0, k[5] * z, k[5] * y},
        {-2 * k[6] * x, -2 * k[6] * y, 4 * k[6] * z},
        {k[7] * z, 0, k[7] * x},
        {2 * k[8] * x, -2 * k[8] * y, 0},
        {6 * k[9] * x * y, k[9] * (3 * xx - 3 * yy), 0},
        {k[10] * y * z, k[10] * x * z, k[10] * x * y},
        {-2 * k[11] * x * y, k[11] * (4 * zz - xx - 3 * yy), 8 * k[11] * y * z},
        {-6 * k[12] * x * z, -6 * k[12] * y * z, k[12] * (6 * zz - 3 * xx - 3 * yy)},
        {k[13] * (4 * zz - 3 * xx - yy), -2 * k[13] * x * y, 8 * k[13] * x * z},
        {2 * k[14] * x * z, -2 * k[14] * y * z, k[14] * (xx - yy)},
        {k[15] * (3 * xx - 3 * yy), -6 * k[15] * x * y, 0},
    };
    for (int i = 0; i < 16; ++i)
        for (int j = 0; j < 3; ++j) dY[i][j] = g[i][j];
}

// Backward of project_gaussian for one Gaussian, in double, by the chain
// rule the "rigel" README "Backward" section lays out for its projection
// backward: from dL/d(u, v) and dL/d(A, B, C) through the 2x2 inverse, through
// Sigma_2d = T Sigma T^T with T = J W, through J's dependence on the camera-
// space centre (a clamped x/z or y/z sends its gradient to z only), through
// the pinhole and the camera transform to the mean; through Sigma = M M^T,
// M = R(q) S to the scales and the normalised quaternion, and through the
// normalisation to the raw quaternion ("Deliberate differences": the
// quaternion normalisation is part of the backward). The colour gradient
// reaches the SH coefficients and, through the view direction
// normalize(mean - campos), the mean ([zenn] 2.2.3 basis).
// clamp_x / clamp_y: which branch the forward took (decided in fp32).
struct Grad3d {
    double mean[3], scale[3], quat[4], sh[48], rgb[3];
};

void project_bwd(const orc_camera* cam, const double m[3], const double s3[3], const double q[4],
                 const double* sh_g, int n_coef, bool clamp_x, bool clamp_y, const double dL_duv[2],
                 const double dL_dconic[3], const double dL_dcol[3], Grad3d* out) {
    double W[9];
    for (int i = 0; i < 9; ++i) W[i] = (double)cam->R[i];
    const double fx = cam->fx, fy = cam->fy;
    // forward quantities
    double p[3];
    for (int i = 0; i < 3; ++i)
        p[i] = W[3 * i + 0] * m[0] + W[3 * i + 1] * m[1] + W[3 * i + 2] * m[2] + (double)cam->t[i];
    const double px = p[0], py = p[1], pz = p[2];
    const double limx = (double)FRUSTUM_CLAMP * ((0.5 * cam->width) / fx);
    const double limy = (double)FRUSTUM_CLAMP * ((0.5 * cam->height) / fy);
    const double Lx = px / pz > 0 ? limx : -limx, Ly = py / pz > 0 ? limy : -limy;
    const double xj = clamp_x ? Lx * pz : px, yj = clamp_y ? Ly * pz : py;
    const double J00 = fx / pz, J02 = -fx * xj / (pz * pz);
    const double J11 = fy / pz, J12 = -fy * yj / (pz * pz);
    const double qn = std::sqrt(q[0] * q[0] + q[1] * q[1] + q[2] * q[2] + q[3] * q[3]);
    const double w = q[0] / qn, x = q[1] / qn, y = q[2] / qn, z = q[3] / qn;
    const double R[3][3] = {
        {1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)},
        {2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)},
        {2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)}};
    double M[3][3], Sig[3][3];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) M[i][j] = R[i][j] * s3[j];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j) Sig[i][j] = M[i][0] * M[j][0] + M[i][1] * M[j][1] + M[i][2] * M[j][2];
    double T[2][3];
    for (int j = 0; j < 3; ++j) {
        T[0][j] = J00 * W[j] + J02 * W[6 + j];
        T[1][j] = J11 * W[3 + j] + J12 * W[6 + j];
    }
    double ST[2][3];  // (Sigma T_r^T) for rows r = 0, 1
    for (int r = 0; r < 2; ++r)
        for (int i = 0; i < 3; ++i) ST[r][i] = Sig[i][0] * T[r][0] + Sig[i][1] * T[r][1] + Sig[i][2] * T[r][2];
    const double a = T[0][0] * ST[0][0] + T[0][1] * ST[0][1] + T[0][2] * ST[0][2] + (double)DILATION;
    const double b = T[0][0] * ST[1][0] + T[0][1] * ST[1][1] + T[0][2] * ST[1][2];
    const double c = T[1][0] * ST[1][0] + T[1][1] * ST[1][1] + T[1][2] * ST[1][2] + (double)DILATION;
    const double det = a * c - b * b, det2 = det * det;

    // conic (A, B, C) = (c, -b, a) / det  ->  Sigma_2d entries
    const double gA = dL_dconic[0], gB = dL_dconic[1], gC = dL_dconic[2];
    const double ga = (-c * c * gA + b * c * gB - b * b * gC) / det2;
    const double gb = (2 * b * c * gA - (a * c + b * b) * gB + 2 * a * b * gC) / det2;
    const double gc = (-b * b * gA + a * b * gB - a * a * gC) / det2;

    // Sigma_2d = T Sigma T^T  ->  T and Sigma
    double gT[2][3];
    for (int j = 0; j < 3; ++j) {
        gT[0][j] = 2 * ga * ST[0][j] + gb * ST[1][j];
        gT[1][j] = gb * ST[0][j] + 2 * gc * ST[1][j];
    }
    double gSig[3][3];  // symmetric part of dL/dSigma
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            gSig[i][j] = ga * T[0][i] * T[0][j] + 0.5 * gb * (T[0][i] * T[1][j] + T[1][i] * T[0][j]) +
                         gc * T[1][i] * T[1][j];

    // T = J W  ->  J
    double gJ00 = 0, gJ02 = 0, gJ11 = 0, gJ12 = 0;
    for (int j = 0; j < 3; ++j) {
        gJ00 += gT[0][j] * W[j];
        gJ02 += gT[0][j] * W[6 + j];
        gJ11 += gT[1][j] * W[3 + j];
        gJ12 += gT[1][j] * W[6 + j];
    }
    // J and the pinhole  ->  camera-space centre
    double gp[3] = {0, 0, 0};
    gp[0] += dL_duv[0] * fx / pz;
    gp[1] += dL_duv[1] * fy / pz;
    gp[2] += -dL_duv[0] * fx * px / (pz * pz) - dL_duv[1] * fy * py / (pz * pz);
    gp[2] += -gJ00 * fx / (pz * pz) - gJ11 * fy / (pz * pz);
    if (clamp_x) {
        gp[2] += gJ02 * fx * Lx / (pz * pz);
    } else {
        gp[0] += -gJ02 * fx / (pz * pz);
        gp[2] += gJ02 * 2 * fx * px / (pz * pz * pz);
    }
    if (clamp_y) {
        gp[2] += gJ12 * fy * Ly / (pz * pz);
    } else {
        gp[1] += -gJ12 * fy / (pz * pz);
        gp[2] += gJ12 * 2 * fy * py / (pz * pz * pz);
    }
    // camera transform p = W m + t  ->  mean
    for (int i = 0; i < 3; ++i) out->mean[i] = W[i] * gp[0] + W[3 + i] * gp[1] + W[6 + i] * gp[2];

    // Sigma = M M^T  ->  M;  M = R S  ->  R and S
    double gM[3][3];
    for (int i = 0; i < 3; ++i)
        for (int j = 0; j < 3; ++j)
            gM[i][j] = 2 * (gSig[i][0] * M[0][j] + gSig[i][1] * M[1][j] + gSig[i][2] * M[2][j]);
    double gR[3][3];
    for (int j = 0; j < 3; ++j) {
        out->scale[j] = gM[0][j] * R[0][j] + gM[1][j] * R[1][j] + gM[2][j] * R[2][j];
        for (int i = 0; i < 3; ++i) gR[i][j] = gM[i][j] * s3[j];
    }
    // R(q) of the normalised quaternion  ->  (w, x, y, z)
    const double gw = 2 * (-z * gR[0][1] + y * gR[0][2] + z * gR[1][0] - x * gR[1][2] - y * gR[2][0] + x * gR[2][1]);
    const double gx = 2 * (y * gR[0][1] + z * gR[0][2] + y * gR[1][0] - 2 * x * gR[1][1] - w * gR[1][2] +
                           z * gR[2][0] + w * gR[2][1] - 2 * x * gR[2][2]);
    const double gy = 2 * (-2 * y * gR[0][0] + x * gR[0][1] + w * gR[0][2] + x * gR[1][0] + z * gR[1][2] -
                           w * gR[2][0] + z * gR[2][1] - 2 * y * gR[2][2]);
    const double gz = 2 * (-2 * z * gR[0][0] - w * gR[0][1] + x * gR[0][2] + w * gR[1][0] - 2 * z * gR[1][1] +
                           y * gR[1][2] + x * gR[2][0] + y * gR[2][1]);
    // normalisation q_hat = q / |q|: remove the radial part, divide by |q|
    const double dot = w * gw + x * gx + y * gy + z * gz;
    out->quat[0] = (gw - w * dot) / qn;
    out->quat[1] = (gx - x * dot) / qn;
    out->quat[2] = (gy - y * dot) / qn;
    out->quat[3] = (gz - z * dot) / qn;

    // colour
    if (sh_g) {
        const double v0 = m[0] - cam->campos[0], v1 = m[1] - cam->campos[1], v2 = m[2] - cam->campos[2];
        const double vn = std::sqrt(v0 * v0 + v1 * v1 + v2 * v2);
        const double d[3] = {v0 / vn, v1 / vn, v2 / vn};
        double Y[16], dY[16][3];
        sh_basis<double>(d[0], d[1], d[2], Y);
        sh_basis_grad(d[0], d[1], d[2], dY);
        double gd[3] = {0, 0, 0};
        for (int k = 0; k < n_coef; ++k)
            for (int ch = 0; ch < 3; ++ch) {
                out->sh[k * 3 + ch] = dL_dcol[ch] * Y[k];
                for (int j = 0; j < 3; ++j) gd[j] += dL_dcol[ch] * sh_g[k * 3 + ch] * dY[k][j];
            }
        const double dd = d[0] * gd[0] + d[1] * gd[1] + d[2] * gd[2];
        for (int j = 0; j < 3; ++j) out->mean[j] += (gd[j] - d[j] * dd) / vn;
    } else {
        for (int ch = 0; ch < 3; ++ch) out->rgb[ch] = dL_dcol[ch];
    }
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

// Preprocess, one Gaussian at a time (project_gaussian in fp32, then the
// tile span). Layouts: means/scales [3][n], quats [4][n] (w,x,y,z), opacity
// [n], sh [(d+1)^2][3][n] or NULL (then rgb_in [3][n]). Outputs per
// Gaussian: xy_depth (u, v, z, radius), conic_op (A, B, C, opacity), rgb
// (r, g, b, 0), tiles_touched. A culled Gaussian gets all-zero outputs; a
// Gaussian whose opacity or colour is not finite is culled as well.
// Returns 0, or -1 on an invalid argument.
int orc_preprocess_ex(const orc_camera* cam, int32_t n, const float* means,
                      const float* scales, const float* quats, const float* opacity,
                      const float* sh, int32_t sh_degree, const float* rgb_in,
                      float* xy_depth, float* conic_op, float* rgb,
                      uint32_t* tiles_touched, int32_t tile_test) {
    if (!cam || n < 0 || tile_test < 0 || tile_test > 1) return -1;
    if (sh && (sh_degree < 0 || sh_degree > 3)) return -1;
    const int TX = tiles_x(cam), TY = tiles_y(cam);
    const int n_coef = sh ? (sh_degree + 1) * (sh_degree + 1) : 0;

#pragma omp parallel for schedule(static) num_threads(g_threads) if (g_threads > 1)
    for (int g = 0; g < n; ++g) {
        float* o_xy = xy_depth + 4 * (size_t)g;
        float* o_co = conic_op + 4 * (size_t)g;
        float* o_rgb = rgb + 4 * (size_t)g;
        for (int k = 0; k < 4; ++k) { o_xy[k] = 0.0f; o_co[k] = 0.0f; o_rgb[k] = 0.0f; }
        tiles_touched[g] = 0;

        float m[3], s3[3], q[4], sh_g[48], rgb_g[3];
        gather_gaussian<float, float>(n, g, means, scales, quats, sh, n_coef, sh ? nullptr : rgb_in,
                                      m, s3, q, sh_g, rgb_g);
        Projected<float> P;
        if (!project_gaussian<float>(cam, m, s3, q, sh ? sh_g : nullptr, n_coef, rgb_g, &P)) continue;

        // Tile span; nothing on screen means culled. With the ellipse test,
        // only the tiles it keeps are counted (none kept: culled).
        const Span sp = tile_span(P.u, P.v, P.r, TX, TY);
        int count = (sp.x1 - sp.x0) * (sp.y1 - sp.y0);
        if (count > 0 && tile_test == 1) {
            const EllipseRows er = ellipse_rows(P.u, P.v, P.A, P.B, P.C, sp);
            count = 0;
            for (int ty = sp.y0; ty < sp.y1; ++ty) {
                int lo, hi;
                ellipse_row_range(er, sp, ty, &lo, &hi);
                count += hi > lo ? hi - lo : 0;
            }
        }
        if (count <= 0) continue;
        if (!std::isfinite(opacity[g]) || !std::isfinite(P.col[0]) || !std::isfinite(P.col[1]) ||
            !std::isfinite(P.col[2])) continue;

        o_xy[0] = P.u; o_xy[1] = P.v; o_xy[2] = P.z; o_xy[3] = P.r;
        o_co[0] = P.A; o_co[1] = P.B; o_co[2] = P.C; o_co[3] = opacity[g];
        o_rgb[0] = P.col[0]; o_rgb[1] = P.col[1]; o_rgb[2] = P.col[2];
        tiles_touched[g] = (uint32_t)count;
    }
    return 0;
}

// Backward of orc_preprocess (the projection backward of the "rigel" README
// "Backward" section, plus the SH colour). The cull and the clamp branches
// are decided by the fp32 preprocess exactly as orc_preprocess decides
// them; the derivatives are evaluated in double at the fp32 inputs. A
// culled Gaussian gets zero gradients.
// In:  grad_mean2d [n][2] (du, dv), grad_conic_op [n][4] (dA, dB, dC,
//      dopacity), grad_rgb [n][4] (dr, dg, db, -), all double.
// Out: grad_means [3][n], grad_scales [3][n], grad_quats [4][n],
//      grad_opacity [n], and grad_sh [(d+1)^2][3][n] when sh != NULL, else
//      grad_rgb_in [3][n]. Everything is overwritten. Returns 0, or -1 on an
//      invalid argument.
int orc_preprocess_bwd(const orc_camera* cam, int32_t n, const float* means, const float* scales,
                       const float* quats, const float* opacity, const float* sh, int32_t sh_degree,
                       const float* rgb_in, const double* grad_mean2d, const double* grad_conic_op,
                       const double* grad_rgb, double* grad_means, double* grad_scales,
                       double* grad_quats, double* grad_opacity, double* grad_sh,
                       double* grad_rgb_in) {
    if (!cam || n < 0) return -1;
    if (sh && (sh_degree < 0 || sh_degree > 3)) return -1;
    const int TX = tiles_x(cam), TY = tiles_y(cam);
    const int n_coef = sh ? (sh_degree + 1) * (sh_degree + 1) : 0;
    for (int g = 0; g < n; ++g) {
        for (int i = 0; i < 3; ++i) { grad_means[(size_t)i * n + g] = 0; grad_scales[(size_t)i * n + g] = 0; }
        for (int i = 0; i < 4; ++i) grad_quats[(size_t)i * n + g] = 0;
        grad_opacity[g] = 0;
        if (sh) {
            for (int k = 0; k < 3 * n_coef; ++k) grad_sh[(size_t)k * n + g] = 0;
        } else {
            for (int ch = 0; ch < 3; ++ch) grad_rgb_in[(size_t)ch * n + g] = 0;
        }
        // the forward's decisions, in fp32
        float m[3], s3[3], q[4], sh_g[48], rgb_g[3];
        gather_gaussian<float, float>(n, g, means, scales, quats, sh, n_coef, sh ? nullptr : rgb_in,
                                      m, s3, q, sh_g, rgb_g);
        Projected<float> P;
        if (!project_gaussian<float>(cam, m, s3, q, sh ? sh_g : nullptr, n_coef, rgb_g, &P)) continue;
        const Span sp = tile_span(P.u, P.v, P.r, TX, TY);
        if ((sp.x1 - sp.x0) * (sp.y1 - sp.y0) <= 0) continue;
        if (!std::isfinite(opacity[g]) || !std::isfinite(P.col[0]) || !std::isfinite(P.col[1]) ||
            !std::isfinite(P.col[2])) continue;
        // the derivatives, in double
        double md[3], sd[3], qd[4], shd[48], rgbd[3];
        gather_gaussian<double, float>(n, g, means, scales, quats, sh, n_coef, sh ? nullptr : rgb_in,
                                       md, sd, qd, shd, rgbd);
        const double duv[2] = {grad_mean2d[2 * (size_t)g], grad_mean2d[2 * (size_t)g + 1]};
        const double dcon[3] = {grad_conic_op[4 * (size_t)g], grad_conic_op[4 * (size_t)g + 1],
                                grad_conic_op[4 * (size_t)g + 2]};
        const double dcol[3] = {grad_rgb[4 * (size_t)g], grad_rgb[4 * (size_t)g + 1], grad_rgb[4 * (size_t)g + 2]};
        Grad3d G;
        project_bwd(cam, md, sd, qd, sh ? shd : nullptr, n_coef, P.clamp_x, P.clamp_y, duv, dcon, dcol, &G);
        for (int i = 0; i < 3; ++i) { grad_means[(size_t)i * n + g] = G.mean[i]; grad_scales[(size_t)i * n + g] = G.scale[i]; }
        for (int i = 0; i < 4; ++i) grad_quats[(size_t)i * n + g] = G.quat[i];
        grad_opacity[g] = grad_conic_op[4 * (size_t)g + 3];
        if (sh) {
            for (int k = 0; k < 3 * n_coef; ++k) grad_sh[(size_t)k * n + g] = G.sh[k];
        } else {
            for (int ch = 0; ch < 3; ++ch) grad_rgb_in[(size_t)ch * n + g] = G.rgb[ch];
        }
    }
    return 0;
}

// project_gaussian in double for one Gaussian (the function whose finite
// differences pin orc_preprocess_bwd). Inputs in double: m[3], s[3], q[4],
// sh_g [n_coef][3] (or NULL with rgb_g[3]). out[0..9] = u, v, A, B, C,
// r, g, b, clamp_x, clamp_y. Returns 1, or 0 when culled.
int orc_project_f64(const orc_camera* cam, const double* m, const double* s3, const double* q,
                    const double* sh_g, int32_t n_coef, const double* rgb_g, double* out) {
    Projected<double> P;
    if (!project_gaussian<double>(cam, m, s3, q, sh_g, n_coef, rgb_g, &P)) return 0;
    out[0] = P.u; out[1] = P.v; out[2] = P.A; out[3] = P.B; out[4] = P.C;
    out[5] = P.col[0]; out[6] = P.col[1]; out[7] = P.col[2];
    out[8] = P.clamp_x ? 1.0 : 0.0; out[9] = P.clamp_y ? 1.0 : 0.0;
    return 1;
}

int orc_preprocess(const orc_camera* cam, int32_t n, const float* means,
                   const float* scales, const float* quats, const float* opacity,
                   const float* sh, int32_t sh_degree, const float* rgb_in,
                   float* xy_depth, float* conic_op, float* rgb,
                   uint32_t* tiles_touched) {
    return orc_preprocess_ex(cam, n, means, scales, quats, opacity, sh, sh_degree, rgb_in, xy_depth,
                             conic_op, rgb, tiles_touched, 0);
}

// Kept tile range [lo, hi) of row ty for one splat under the ellipse test
// (exposed for the pins): out = lo, hi.
void orc_ellipse_row_range(float u, float v, float r, float A, float B, float C, int32_t TX,
                           int32_t TY, int32_t ty, int32_t* out) {
    const Span sp = tile_span(u, v, r, TX, TY);
    const EllipseRows er = ellipse_rows(u, v, A, B, C, sp);
    int lo, hi;
    ellipse_row_range(er, sp, ty, &lo, &hi);
    out[0] = lo; out[1] = hi;
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
// With tile_test == 1 (conic_op given) only the tiles the ellipse test
// keeps are written, in the same order.
int orc_duplicate_ex(const orc_camera* cam, int32_t n, const float* xy_depth, const float* conic_op,
                     const uint32_t* tiles_touched, const uint64_t* offsets,
                     uint64_t* keys, uint32_t* values, int32_t tile_test) {
    const int TX = tiles_x(cam), TY = tiles_y(cam);
    for (int g = 0; g < n; ++g) {
        if (tiles_touched[g] == 0) continue;
        const float* rec = xy_depth + 4 * (size_t)g;
        const Span sp = tile_span(rec[0], rec[1], rec[3], TX, TY);
        const uint64_t depth_bits = float_bits(rec[2]);
        const uint64_t k0 = offsets[g];
        uint64_t k = k0;
        if (tile_test == 1) {
            const float* co = conic_op + 4 * (size_t)g;
            const EllipseRows er = ellipse_rows(rec[0], rec[1], co[0], co[1], co[2], sp);
            for (int ty = sp.y0; ty < sp.y1; ++ty) {
                int lo, hi;
                ellipse_row_range(er, sp, ty, &lo, &hi);
                for (int tx = lo; tx < hi; ++tx) {
                    if (k - k0 >= tiles_touched[g]) return -2;
                    keys[k] = ((uint64_t)(ty * TX + tx) << 32) | depth_bits;
                    values[k] = (uint32_t)g;
                    ++k;
                }
            }
        } else {
            if ((uint32_t)((sp.x1 - sp.x0) * (sp.y1 - sp.y0)) != tiles_touched[g]) return -2;
            for (int ty = sp.y0; ty < sp.y1; ++ty)
                for (int tx = sp.x0; tx < sp.x1; ++tx) {
                    keys[k] = ((uint64_t)(ty * TX + tx) << 32) | depth_bits;
                    values[k] = (uint32_t)g;
                    ++k;
                }
        }
        if (k - k0 != tiles_touched[g]) return -2;
    }
    return 0;
}

int orc_duplicate(const orc_camera* cam, int32_t n, const float* xy_depth,
                  const uint32_t* tiles_touched, const uint64_t* offsets,
                  uint64_t* keys, uint32_t* values) {
    return orc_duplicate_ex(cam, n, xy_depth, nullptr, tiles_touched, offsets, keys, values, 0);
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
int64_t orc_bin_ex(const orc_camera* cam, int32_t n, const float* xy_depth, const float* conic_op,
                   const uint32_t* tiles_touched, uint64_t* keys, uint32_t* point_list,
                   int64_t capacity, int32_t tile_test) {
    if (!cam || n < 0 || tile_test < 0 || tile_test > 1 || (tile_test == 1 && !conic_op)) return -1;
    std::vector<uint64_t> offsets((size_t)n);
    const uint64_t total = orc_exclusive_scan(tiles_touched, n, offsets.data());
    if ((int64_t)total > capacity) return (int64_t)total;
    if (orc_duplicate_ex(cam, n, xy_depth, conic_op, tiles_touched, offsets.data(), keys, point_list,
                         tile_test) != 0)
        return -2;
    orc_sort_pairs(keys, point_list, (int64_t)total);
    return (int64_t)total;
}

int64_t orc_bin(const orc_camera* cam, int32_t n, const float* xy_depth,
                const uint32_t* tiles_touched, uint64_t* keys, uint32_t* point_list,
                int64_t capacity) {
    return orc_bin_ex(cam, n, xy_depth, nullptr, tiles_touched, keys, point_list, capacity, 0);
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
#pragma omp parallel for schedule(dynamic, 4) num_threads(g_threads) if (g_threads > 1)
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

// The backward's walk over pixel rows [y0, y1), adding each term to the
// given gradient arrays (and its magnitude to mass_* when those are given).
template <typename F>
void composite_bwd_rows(const orc_camera* cam, const uint32_t* ranges, const uint32_t* point_list,
                        const F* xy_depth, const F* conic_op, const F* rgb, const F* bg, const F* final_T,
                        const uint32_t* n_contrib, const F* dL_dimage, int y0, int y1, double* grad_mean2d,
                        double* grad_conic_op, double* grad_rgb, double* mass_mean2d, double* mass_conic_op,
                        double* mass_rgb) {
    const int Wd = cam->width, Hd = cam->height, TX = tiles_x(cam);
    const F alpha_min = (F)ALPHA_MIN, alpha_max = (F)ALPHA_MAX;
    const bool mass = mass_mean2d && mass_conic_op && mass_rgb;
    // adds a term to a gradient element (and its magnitude to the mass)
    auto add = [&](double* grad, double* m, size_t i, F term) {
        grad[i] += (double)term;
        if (mass) m[i] += std::fabs((double)term);
    };
    for (int y = y0; y < y1; ++y) {
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
                    add(grad_rgb, mass_rgb, 4 * (size_t)g + ch, a * Tj * gpix[ch]);
                    dL_da = dL_da + gpix[ch] * (c[ch] - B[ch]);
                }
                dL_da = dL_da * Tj;
                for (int ch = 0; ch < 3; ++ch) B[ch] = a * c[ch] + ((F)1 - a) * B[ch];
                T = Tj;
                if (a_raw > alpha_max) continue;  // saturated: no gradient to o, conic, mean
                const F dp = a * dL_da;
                add(grad_conic_op, mass_conic_op, 4 * (size_t)g + 3, G * dL_da);
                add(grad_conic_op, mass_conic_op, 4 * (size_t)g + 0, (F)(-0.5) * dx * dx * dp);
                add(grad_conic_op, mass_conic_op, 4 * (size_t)g + 1, -dx * dy * dp);
                add(grad_conic_op, mass_conic_op, 4 * (size_t)g + 2, (F)(-0.5) * dy * dy * dp);
                add(grad_mean2d, mass_mean2d, 2 * (size_t)g + 0, (co[0] * dx + co[1] * dy) * dp);
                add(grad_mean2d, mass_mean2d, 2 * (size_t)g + 1, (co[1] * dx + co[2] * dy) * dp);
            }
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
// Optionally (mass_* non-NULL) also the per-element sum over pixels of the
// magnitudes of the terms each gradient is summed from, the scale against
// which a float32 sum with cancellation is judged.
template <typename F>
void composite_bwd(const orc_camera* cam, int32_t n, const uint32_t* ranges,
                   const uint32_t* point_list, const F* xy_depth, const F* conic_op,
                   const F* rgb, const F* bg, const F* final_T, const uint32_t* n_contrib,
                   const F* dL_dimage, double* grad_mean2d, double* grad_conic_op,
                   double* grad_rgb, double* mass_mean2d = nullptr, double* mass_conic_op = nullptr,
                   double* mass_rgb = nullptr) {
    const int Hd = cam->height;
    const bool mass = mass_mean2d && mass_conic_op && mass_rgb;
    double* outs[6] = {grad_mean2d, grad_conic_op, grad_rgb, mass_mean2d, mass_conic_op, mass_rgb};
    const size_t len[6] = {2 * (size_t)n, 4 * (size_t)n, 4 * (size_t)n, 2 * (size_t)n, 4 * (size_t)n,
                           4 * (size_t)n};
    for (int k = 0; k < (mass ? 6 : 3); ++k) std::fill(outs[k], outs[k] + len[k], 0.0);
    const int T = std::max(1, std::min(g_threads, Hd));
    if (T == 1) {
        composite_bwd_rows<F>(cam, ranges, point_list, xy_depth, conic_op, rgb, bg, final_T, n_contrib, dL_dimage,
                              0, Hd, grad_mean2d, grad_conic_op, grad_rgb, mass_mean2d, mass_conic_op, mass_rgb);
        return;
    }
    // thread t: rows [t Hd / T, (t + 1) Hd / T) into its own arrays, summed in thread order
    const size_t per = 10 * (size_t)n;
    std::vector<double> part((size_t)T * per * (mass ? 2 : 1), 0.0);
#pragma omp parallel for schedule(static, 1) num_threads(T)
    for (int t = 0; t < T; ++t) {
        double* b = part.data() + (size_t)t * per * (mass ? 2 : 1);
        double* m = mass ? b + per : nullptr;
        composite_bwd_rows<F>(cam, ranges, point_list, xy_depth, conic_op, rgb, bg, final_T, n_contrib, dL_dimage,
                              (int)((int64_t)t * Hd / T), (int)((int64_t)(t + 1) * Hd / T), b, b + 2 * (size_t)n,
                              b + 6 * (size_t)n, m, m ? m + 2 * (size_t)n : nullptr, m ? m + 6 * (size_t)n : nullptr);
    }
    for (int t = 0; t < T; ++t) {
        const double* b = part.data() + (size_t)t * per * (mass ? 2 : 1);
        for (int k = 0; k < (mass ? 6 : 3); ++k) {
            const double* src = b + (k >= 3 ? per : 0) + (k % 3 == 0 ? 0 : (k % 3 == 1 ? 2 * (size_t)n : 6 * (size_t)n));
            for (size_t i = 0; i < len[k]; ++i) outs[k][i] += src[i];
        }
    }
}

}  // namespace

extern "C" {

// Threads for the preprocess and the compositing (see g_threads); values
// below 1 mean 1. Returns the number set.
int orc_set_threads(int32_t threads) {
    g_threads = std::max(1, (int)threads);
    return g_threads;
}

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

// orc_composite_bwd_f32 plus the per-element term magnitudes (mass_*,
// laid out as the gradients).
void orc_composite_bwd_mass_f32(const orc_camera* cam, int32_t n, const uint32_t* ranges,
                                const uint32_t* point_list, const float* xy_depth, const float* conic_op,
                                const float* rgb, const float* bg, const float* final_T,
                                const uint32_t* n_contrib, const float* dL_dimage, double* grad_mean2d,
                                double* grad_conic_op, double* grad_rgb, double* mass_mean2d,
                                double* mass_conic_op, double* mass_rgb) {
    composite_bwd<float>(cam, n, ranges, point_list, xy_depth, conic_op, rgb, bg, final_T, n_contrib,
                         dL_dimage, grad_mean2d, grad_conic_op, grad_rgb, mass_mean2d, mass_conic_op, mass_rgb);
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
