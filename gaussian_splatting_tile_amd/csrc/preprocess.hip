// Preprocess: one thread per Gaussian, structure-of-arrays loads (each
// component read by consecutive lanes from consecutive addresses), packed
// float4 stores.
//
// Follows "rigel" README "Projection"; zenn sections 2.1.1 (Sigma = R S S^T
// R^T), 2.1.2 (the pinhole Jacobian J and Sigma' = J W Sigma W^T J^T), 2.2.3
// (SH basis), 2.3.1 (conic), 2.3.3 (radius from lambda_max); learn-gs
// prep_splats (near cull, det > 0) and tile_spans.
//
// Everything is float32 with a fixed operation order and no contraction
// (the library is built with -ffp-contract=off; division and square root
// are correctly rounded), so every output is reproducible bit for bit by a
// host evaluation of the same formulas. That is what lets the integer
// results downstream (radius, tile span, sort keys) match exactly.
#include "gs_internal.h"

namespace gs {
namespace {

// Real SH constants (closed forms of the zenn 2.2.3 table, Sloan's
// polynomial forms), rounded to float from 17 significant digits.
constexpr float kSh0 = 0.28209479177387814f;   // 1 / (2 sqrt(pi))
constexpr float kSh1 = 0.4886025119029199f;    // sqrt(3 / (4 pi))
constexpr float kSh2a = 1.0925484305920792f;   // sqrt(15 / pi) / 2
constexpr float kSh2b = 0.31539156525252005f;  // sqrt(5 / pi) / 4
constexpr float kSh2c = 0.5462742152960396f;   // sqrt(15 / pi) / 4
constexpr float kSh3a = 0.5900435899266435f;   // sqrt(35 / (2 pi)) / 4
constexpr float kSh3b = 2.890611442640554f;    // sqrt(105 / pi) / 2
constexpr float kSh3c = 0.4570457994644658f;   // sqrt(21 / (2 pi)) / 4
constexpr float kSh3d = 0.3731763325901154f;   // sqrt(7 / pi) / 4
constexpr float kSh3e = 1.445305721320277f;    // sqrt(105 / pi) / 4

// The splat record of Gaussian g seen by camera cam. The Gaussian's inputs
// come from `in` (in.mean(c), in.quat(c), in.scale(c), in.opacity(),
// in.sh(row), in.rgb(c)), read only once the splat survives the culls
// before them; outputs are (0, 0, 0, 0) records and count 0 when culled.
template <class In>
__device__ __forceinline__ void project_splat(const gs_camera& cam, const In& in, const bool has_sh, const int n_coef,
                                              const uint32_t flags, float4& o_xy, float4& o_co, float4& o_rgb,
                                              uint32_t& count) {
    const int TX = (cam.width + kTile - 1) / kTile;
    const int TY = (cam.height + kTile - 1) / kTile;
    const float* W = cam.R;

    o_xy = make_float4(0.f, 0.f, 0.f, 0.f);
    o_co = o_xy;
    o_rgb = o_xy;
    count = 0;

    do {
        const float mx = in.mean(0), my = in.mean(1), mz = in.mean(2);

        // World to camera.
        const float px = ((W[0] * mx + W[1] * my) + W[2] * mz) + cam.t[0];
        const float py = ((W[3] * mx + W[4] * my) + W[5] * mz) + cam.t[1];
        const float pz = ((W[6] * mx + W[7] * my) + W[8] * mz) + cam.t[2];
        if (!(pz > kZNear)) break;

        // Pinhole centre.
        const float u = (cam.fx * px) / pz + cam.cx;
        const float v = (cam.fy * py) / pz + cam.cy;
        if (!isfinite(u) || !isfinite(v)) break;

        // Jacobian at the centre with x/z, y/z clamped to 1.3x the half-width.
        const float limx = kFrustumClamp * ((0.5f * (float)cam.width) / cam.fx);
        const float limy = kFrustumClamp * ((0.5f * (float)cam.height) / cam.fy);
        const float xj = fminf(limx, fmaxf(-limx, px / pz)) * pz;
        const float yj = fminf(limy, fmaxf(-limy, py / pz)) * pz;
        const float zz = pz * pz;
        const float J00 = cam.fx / pz;
        const float J02 = -(cam.fx * xj) / zz;
        const float J11 = cam.fy / pz;
        const float J12 = -(cam.fy * yj) / zz;

        // Normalised quaternion (w, x, y, z) to rotation.
        float qw = in.quat(0), qx = in.quat(1), qy = in.quat(2), qz = in.quat(3);
        const float qn = sqrtf(((qw * qw + qx * qx) + qy * qy) + qz * qz);
        if (!(qn > 0.0f)) break;
        qw = qw / qn;
        qx = qx / qn;
        qy = qy / qn;
        qz = qz / qn;
        const float r00 = 1.0f - 2.0f * (qy * qy + qz * qz);
        const float r01 = 2.0f * (qx * qy - qw * qz);
        const float r02 = 2.0f * (qx * qz + qw * qy);
        const float r10 = 2.0f * (qx * qy + qw * qz);
        const float r11 = 1.0f - 2.0f * (qx * qx + qz * qz);
        const float r12 = 2.0f * (qy * qz - qw * qx);
        const float r20 = 2.0f * (qx * qz - qw * qy);
        const float r21 = 2.0f * (qy * qz + qw * qx);
        const float r22 = 1.0f - 2.0f * (qx * qx + qy * qy);

        // M = R(q) S, Sigma = M M^T (symmetric; six distinct entries).
        const float sx = in.scale(0), sy = in.scale(1), sz = in.scale(2);
        const float m00 = r00 * sx, m01 = r01 * sy, m02 = r02 * sz;
        const float m10 = r10 * sx, m11 = r11 * sy, m12 = r12 * sz;
        const float m20 = r20 * sx, m21 = r21 * sy, m22 = r22 * sz;
        const float s00 = (m00 * m00 + m01 * m01) + m02 * m02;
        const float s01 = (m00 * m10 + m01 * m11) + m02 * m12;
        const float s02 = (m00 * m20 + m01 * m21) + m02 * m22;
        const float s11 = (m10 * m10 + m11 * m11) + m12 * m12;
        const float s12 = (m10 * m20 + m11 * m21) + m12 * m22;
        const float s22 = (m20 * m20 + m21 * m21) + m22 * m22;

        // T = J W (J's zeros skipped); U = T Sigma; Sigma_2d = U T^T + 0.3 I.
        const float t00 = J00 * W[0] + J02 * W[6];
        const float t01 = J00 * W[1] + J02 * W[7];
        const float t02 = J00 * W[2] + J02 * W[8];
        const float t10 = J11 * W[3] + J12 * W[6];
        const float t11 = J11 * W[4] + J12 * W[7];
        const float t12 = J11 * W[5] + J12 * W[8];
        const float u00 = (t00 * s00 + t01 * s01) + t02 * s02;
        const float u01 = (t00 * s01 + t01 * s11) + t02 * s12;
        const float u02 = (t00 * s02 + t01 * s12) + t02 * s22;
        const float u10 = (t10 * s00 + t11 * s01) + t12 * s02;
        const float u11 = (t10 * s01 + t11 * s11) + t12 * s12;
        const float u12 = (t10 * s02 + t11 * s12) + t12 * s22;
        const float a = ((u00 * t00 + u01 * t01) + u02 * t02) + kDilation;
        const float b = (u00 * t10 + u01 * t11) + u02 * t12;
        const float c = ((u10 * t10 + u11 * t11) + u12 * t12) + kDilation;
        if (!isfinite(a) || !isfinite(b) || !isfinite(c)) break;

        // Conic; degenerate or non-finite determinants are culled.
        const float det = a * c - b * b;
        if (!(det > 0.0f) || !isfinite(det)) break;
        const float cA = c / det, cB = -b / det, cC = a / det;

        // Radius: 3 sqrt(lambda_max) with the discriminant floored at 0.1.
        const float mid = 0.5f * (a + c);
        const float lam = mid + sqrtf(fmaxf(mid * mid - det, kDiscFloor));
        const float r = ceilf(kSigma * sqrtf(lam));
        if (!isfinite(r)) break;

        const Span sp = tile_span(u, v, r, TX, TY);
        int cnt = (sp.x1 - sp.x0) * (sp.y1 - sp.y0);
        if (cnt > 0 && (flags & kTilesEllipse)) {  // count only the tiles the ellipse test keeps
            const EllipseRows er = ellipse_rows(u, v, cA, cB, cC, sp);
            cnt = 0;
            for (int ty = sp.y0; ty < sp.y1; ++ty) {
                int lo, hi;
                ellipse_row_range(er, sp, ty, lo, hi);
                cnt += hi > lo ? hi - lo : 0;
            }
        }
        if (cnt <= 0) break;

        // Colour.
        float col0, col1, col2;
        if (has_sh) {
            float dx = mx - cam.campos[0], dy = my - cam.campos[1], dz = mz - cam.campos[2];
            const float dn = sqrtf((dx * dx + dy * dy) + dz * dz);
            const float x = dx / dn, y = dy / dn, z = dz / dn;
            const float xx = x * x, yy = y * y, zz2 = z * z;
            float Y[16];
            Y[0] = kSh0;
            Y[1] = -kSh1 * y;
            Y[2] = kSh1 * z;
            Y[3] = -kSh1 * x;
            Y[4] = kSh2a * (x * y);
            Y[5] = -kSh2a * (y * z);
            Y[6] = kSh2b * ((2.0f * zz2 - xx) - yy);
            Y[7] = -kSh2a * (z * x);
            Y[8] = kSh2c * (xx - yy);
            Y[9] = -kSh3a * ((3.0f * xx - yy) * y);
            Y[10] = kSh3b * ((x * y) * z);
            Y[11] = -kSh3c * (((4.0f * zz2 - xx) - yy) * y);
            Y[12] = kSh3d * (z * ((2.0f * zz2 - 3.0f * xx) - 3.0f * yy));
            Y[13] = -kSh3c * (x * ((4.0f * zz2 - xx) - yy));
            Y[14] = kSh3e * ((xx - yy) * z);
            Y[15] = -kSh3a * (x * (xx - 3.0f * yy));
            col0 = in.sh(0) * Y[0];
            col1 = in.sh(1) * Y[0];
            col2 = in.sh(2) * Y[0];
#pragma unroll
            for (int k = 1; k < 16; ++k) {
                if (k < n_coef) {
                    col0 = col0 + in.sh(3 * k + 0) * Y[k];
                    col1 = col1 + in.sh(3 * k + 1) * Y[k];
                    col2 = col2 + in.sh(3 * k + 2) * Y[k];
                }
            }
        } else {
            col0 = in.rgb(0);
            col1 = in.rgb(1);
            col2 = in.rgb(2);
        }
        const float op = in.opacity();
        if (!isfinite(op) || !isfinite(col0) || !isfinite(col1) || !isfinite(col2)) break;

        o_xy = make_float4(u, v, pz, r);
        o_co = make_float4(cA, cB, cC, op);
        o_rgb = make_float4(col0, col1, col2, 0.0f);
        count = (uint32_t)cnt;
    } while (false);
}

// Inputs read from the SoA arrays where the projection needs them: a
// culled Gaussian never loads its SH rows.
struct GlobalIn {
    const float* __restrict__ means;
    const float* __restrict__ scales;
    const float* __restrict__ quats;
    const float* __restrict__ opac;
    const float* __restrict__ shs;
    const float* __restrict__ rgbs;
    size_t n, g;
    __device__ float mean(int c) const { return means[c * n + g]; }
    __device__ float scale(int c) const { return scales[c * n + g]; }
    __device__ float quat(int c) const { return quats[c * n + g]; }
    __device__ float opacity() const { return opac[g]; }
    __device__ float sh(int row) const { return shs[row * n + g]; }
    __device__ float rgb(int c) const { return rgbs[c * n + g]; }
};

// One Gaussian's inputs, held in registers (see load_inputs).
struct RegIn {
    float m[3], s[3], q[4], o, c[48];
    __device__ float mean(int i) const { return m[i]; }
    __device__ float scale(int i) const { return s[i]; }
    __device__ float quat(int i) const { return q[i]; }
    __device__ float opacity() const { return o; }
    __device__ float sh(int row) const { return c[row]; }
    __device__ float rgb(int i) const { return c[i]; }
};

template <int R>
__device__ __forceinline__ void load_rows(float* c, const float* __restrict__ src, int n, int g) {
#pragma unroll
    for (int row = 0; row < R; ++row) c[row] = src[(size_t)row * n + g];
}

// Every input of Gaussian g, loaded at once: the loads are independent, so
// issuing them together costs one memory round trip instead of one per group
// of values as the projection reaches them (the SH coefficients alone are
// sixteen groups). One straight run of loads per SH degree.
__device__ __forceinline__ void load_inputs(RegIn& in, int n, int g, const float* __restrict__ means,
                                            const float* __restrict__ scales, const float* __restrict__ quats,
                                            const float* __restrict__ opacity, const float* __restrict__ sh,
                                            int n_coef, const float* __restrict__ rgb_in) {
    load_rows<3>(in.m, means, n, g);
    load_rows<3>(in.s, scales, n, g);
    load_rows<4>(in.q, quats, n, g);
    in.o = opacity[g];
    if (!sh) load_rows<3>(in.c, rgb_in, n, g);
    else if (n_coef == 16) load_rows<48>(in.c, sh, n, g);
    else if (n_coef == 9) load_rows<27>(in.c, sh, n, g);
    else if (n_coef == 4) load_rows<12>(in.c, sh, n, g);
    else load_rows<3>(in.c, sh, n, g);
}

// Splats per launch below which the single-camera projection loads every
// input up front: too few waves to hide one wave's chain of memory round
// trips (1080p / 160k: 14.5 -> 13.2 us). Above it the launch is bandwidth-
// bound and loading where needed skips culled Gaussians' SH rows.
constexpr int kUpfrontMaxN = 1 << 19;

template <bool kUpfront>
__global__ __launch_bounds__(256) void k_preprocess(
    const gs_camera cam, const int n, const float* __restrict__ means,
    const float* __restrict__ scales, const float* __restrict__ quats,
    const float* __restrict__ opacity, const float* __restrict__ sh, const int n_coef,
    const float* __restrict__ rgb_in, float4* __restrict__ xy_depth, float4* __restrict__ conic_op,
    float4* __restrict__ rgb_out, uint32_t* __restrict__ tiles_touched, const uint32_t flags) {
    const int g = blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= n) return;
    float4 o_xy, o_co, o_rgb;
    uint32_t count;
    if (kUpfront) {
        RegIn in;
        load_inputs(in, n, g, means, scales, quats, opacity, sh, n_coef, rgb_in);
        project_splat(cam, in, sh != nullptr, n_coef, flags, o_xy, o_co, o_rgb, count);
    } else {
        const GlobalIn in{means, scales, quats, opacity, sh, rgb_in, (size_t)n, (size_t)g};
        project_splat(cam, in, sh != nullptr, n_coef, flags, o_xy, o_co, o_rgb, count);
    }
    xy_depth[g] = o_xy;
    conic_op[g] = o_co;
    rgb_out[g] = o_rgb;
    tiles_touched[g] = count;
}

// One thread per Gaussian for a stack of cameras: the Gaussian's inputs are
// read once, its record for camera v lands at v n + g.
__global__ __launch_bounds__(256) void k_preprocess_views(
    const CameraSet cams, const int n, const float* __restrict__ means,
    const float* __restrict__ scales, const float* __restrict__ quats,
    const float* __restrict__ opacity, const float* __restrict__ sh, const int n_coef,
    const float* __restrict__ rgb_in, float4* __restrict__ xy_depth, float4* __restrict__ conic_op,
    float4* __restrict__ rgb_out, uint32_t* __restrict__ tiles_touched, const uint32_t flags) {
    const int g = blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= n) return;
    RegIn in;
    load_inputs(in, n, g, means, scales, quats, opacity, sh, n_coef, rgb_in);
    for (int v = 0; v < cams.n; ++v) {
        float4 o_xy, o_co, o_rgb;
        uint32_t count;
        project_splat(cams.cam[v], in, sh != nullptr, n_coef, flags, o_xy, o_co, o_rgb, count);
        const size_t i = (size_t)v * n + g;
        xy_depth[i] = o_xy;
        conic_op[i] = o_co;
        rgb_out[i] = o_rgb;
        tiles_touched[i] = count;
    }
}


}  // namespace

hipError_t launch_preprocess(const gs_camera& cam, int n, const float* means, const float* scales,
                             const float* quats, const float* opacity, const float* sh,
                             int sh_degree, const float* rgb_in, float4* xy_depth,
                             float4* conic_op, float4* rgb, uint32_t* tiles_touched,
                             uint32_t flags, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int n_coef = sh ? (sh_degree + 1) * (sh_degree + 1) : 0;
    const int blocks = (n + 255) / 256;
    if (n <= kUpfrontMaxN)
        hipLaunchKernelGGL(k_preprocess<true>, dim3(blocks), dim3(256), 0, stream, cam, n, means, scales,
                           quats, opacity, sh, n_coef, rgb_in, xy_depth, conic_op, rgb, tiles_touched, flags);
    else
        hipLaunchKernelGGL(k_preprocess<false>, dim3(blocks), dim3(256), 0, stream, cam, n, means, scales,
                           quats, opacity, sh, n_coef, rgb_in, xy_depth, conic_op, rgb, tiles_touched, flags);
    return hipGetLastError();
}

hipError_t launch_preprocess_views(const CameraSet& cams, int n, const float* means, const float* scales,
                                   const float* quats, const float* opacity, const float* sh, int sh_degree,
                                   const float* rgb_in, float4* xy_depth, float4* conic_op, float4* rgb,
                                   uint32_t* tiles_touched, uint32_t flags, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int n_coef = sh ? (sh_degree + 1) * (sh_degree + 1) : 0;
    const int blocks = (n + 255) / 256;
    hipLaunchKernelGGL(k_preprocess_views, dim3(blocks), dim3(256), 0, stream, cams, n, means, scales, quats,
                       opacity, sh, n_coef, rgb_in, xy_depth, conic_op, rgb, tiles_touched, flags);
    return hipGetLastError();
}

}  // namespace gs
