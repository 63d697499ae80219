// Projection + SH backward: one thread per Gaussian, structure-of-arrays
// loads and stores (each component read and written by consecutive lanes at
// consecutive addresses), float32 arithmetic.
//
// Follows the "rigel" README, section "Backward" (its projection backward:
// dL/d means2D and dL/d conic are chained through the 2x2 inverse, through
// Sigma_2d = T Sigma T^T with T = J W, through the Jacobian's dependence on
// the camera-space centre, with a clamped x/z or y/z sending its gradient
// to z alone, through the pinhole and the camera transform, and through
// Sigma = M M^T, M = R(q) S, to the scales and the quaternion), and section
// "Deliberate differences" (the forward normalises the quaternion, so the
// backward includes that normalisation). The colour gradient reaches the SH
// coefficients of zenn section 2.2.3 and, through the view direction
// normalize(mean - campos), the mean.
//
// The forward's decisions are re-derived exactly: a Gaussian with
// tiles_touched == 0 was culled and gets zero gradients, and the clamp
// branches are decided from x/z and y/z evaluated with the operation order
// of the preprocess kernel (bit-identical, so the branch is the one the
// forward took).
#include <type_traits>

#include "gs_internal.h"

namespace gs {
namespace {

// Real SH constants (zenn 2.2.3 table, Sloan's polynomial forms).
constexpr float kY0 = 0.28209479177387814f;   // 1 / (2 sqrt(pi))
constexpr float kY1 = 0.4886025119029199f;    // sqrt(3 / (4 pi))
constexpr float kY2a = 1.0925484305920792f;   // sqrt(15 / pi) / 2
constexpr float kY2b = 0.31539156525252005f;  // sqrt(5 / pi) / 4
constexpr float kY2c = 0.5462742152960396f;   // sqrt(15 / pi) / 4
constexpr float kY3a = 0.5900435899266435f;   // sqrt(35 / (2 pi)) / 4
constexpr float kY3b = 2.890611442640554f;    // sqrt(105 / pi) / 2
constexpr float kY3c = 0.4570457994644658f;   // sqrt(21 / (2 pi)) / 4
constexpr float kY3d = 0.3731763325901154f;   // sqrt(7 / pi) / 4
constexpr float kY3e = 1.445305721320277f;    // sqrt(105 / pi) / 4

__global__ __launch_bounds__(256) void k_preprocess_bwd(
    const gs_camera cam, const int n, const float* __restrict__ means,
    const float* __restrict__ scales, const float* __restrict__ quats,
    const float* __restrict__ sh, const int n_coef, const uint32_t* __restrict__ tiles_touched,
    const float2* __restrict__ grad_mean2d, const float4* __restrict__ grad_conic_op,
    const float4* __restrict__ grad_rgb, float* __restrict__ grad_means,
    float* __restrict__ grad_scales, float* __restrict__ grad_quats,
    float* __restrict__ grad_opacity, float* __restrict__ grad_sh, float* __restrict__ grad_rgb_in) {
    const int g = blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= n) return;
    const size_t N = (size_t)n;

    float gm0 = 0.f, gm1 = 0.f, gm2 = 0.f;   // dL/dmean
    float gs0 = 0.f, gs1 = 0.f, gs2 = 0.f;   // dL/dscale
    float gq0 = 0.f, gq1 = 0.f, gq2 = 0.f, gq3 = 0.f;
    float gop = 0.f;
    float dc0 = 0.f, dc1 = 0.f, dc2 = 0.f;   // dL/dcolour
    float dirx = 0.f, diry = 0.f, dirz = 0.f;

    // Every input first, in one batch of independent loads (one memory
    // round trip instead of one per group of values as the math reaches
    // them); a culled Gaussian's values are loaded but not used. One
    // straight run of loads per SH degree (rows past it are not read).
    const bool visible = tiles_touched[g] != 0u;
    const float mx = means[g], my = means[N + g], mz = means[2 * N + g];
    const float q0 = quats[g], q1 = quats[N + g], q2 = quats[2 * N + g], q3 = quats[3 * N + g];
    const float s[3] = {scales[g], scales[N + g], scales[2 * N + g]};
    const float4 gco = grad_conic_op[g];
    const float2 guv = grad_mean2d[g];
    const float4 gcol = grad_rgb[g];
    float shv[48];
    if (sh != nullptr) {
        const int rows = n_coef == 16 ? 48 : n_coef == 9 ? 27 : n_coef == 4 ? 12 : 3;
        auto load = [&](auto R) {
#pragma unroll
            for (int row = 0; row < decltype(R)::value; ++row) shv[row] = sh[(size_t)row * N + g];
        };
        if (rows == 48) load(std::integral_constant<int, 48>{});
        else if (rows == 27) load(std::integral_constant<int, 27>{});
        else if (rows == 12) load(std::integral_constant<int, 12>{});
        else load(std::integral_constant<int, 3>{});
    }

    if (visible) {
        const float* W = cam.R;
        // Camera space and the clamp decision, in the preprocess's order.
        const float px = ((W[0] * mx + W[1] * my) + W[2] * mz) + cam.t[0];
        const float py = ((W[3] * mx + W[4] * my) + W[5] * mz) + cam.t[1];
        const float pz = ((W[6] * mx + W[7] * my) + W[8] * mz) + cam.t[2];
        const float limx = kFrustumClamp * ((0.5f * (float)cam.width) / cam.fx);
        const float limy = kFrustumClamp * ((0.5f * (float)cam.height) / cam.fy);
        const float rx = px / pz, ry = py / pz;
        const bool cx_on = !(rx >= -limx && rx <= limx);
        const bool cy_on = !(ry >= -limy && ry <= limy);

        const float iz = 1.0f / pz, iz2 = iz * iz;
        const float fx = cam.fx, fy = cam.fy;
        const float Lx = rx > 0.0f ? limx : -limx, Ly = ry > 0.0f ? limy : -limy;
        const float xj = cx_on ? Lx * pz : px, yj = cy_on ? Ly * pz : py;
        const float J00 = fx * iz, J02 = -fx * xj * iz2;
        const float J11 = fy * iz, J12 = -fy * yj * iz2;

        // Normalised quaternion and R(q).
        const float qn = sqrtf(q0 * q0 + q1 * q1 + q2 * q2 + q3 * q3);
        const float iq = 1.0f / qn;
        const float w = q0 * iq, x = q1 * iq, y = q2 * iq, z = q3 * iq;
        float R[3][3];
        R[0][0] = 1.f - 2.f * (y * y + z * z); R[0][1] = 2.f * (x * y - w * z); R[0][2] = 2.f * (x * z + w * y);
        R[1][0] = 2.f * (x * y + w * z); R[1][1] = 1.f - 2.f * (x * x + z * z); R[1][2] = 2.f * (y * z - w * x);
        R[2][0] = 2.f * (x * z - w * y); R[2][1] = 2.f * (y * z + w * x); R[2][2] = 1.f - 2.f * (x * x + y * y);
        float M[3][3];
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j) M[i][j] = R[i][j] * s[j];
        float S[3][3];
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j) S[i][j] = M[i][0] * M[j][0] + M[i][1] * M[j][1] + M[i][2] * M[j][2];

        // T = J W and the rows of Sigma T^T.
        float T0[3], T1[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            T0[j] = J00 * W[j] + J02 * W[6 + j];
            T1[j] = J11 * W[3 + j] + J12 * W[6 + j];
        }
        float P0[3], P1[3];  // Sigma T0^T, Sigma T1^T
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            P0[i] = S[i][0] * T0[0] + S[i][1] * T0[1] + S[i][2] * T0[2];
            P1[i] = S[i][0] * T1[0] + S[i][1] * T1[1] + S[i][2] * T1[2];
        }
        const float a = T0[0] * P0[0] + T0[1] * P0[1] + T0[2] * P0[2] + kDilation;
        const float b = T0[0] * P1[0] + T0[1] * P1[1] + T0[2] * P1[2];
        const float c = T1[0] * P1[0] + T1[1] * P1[1] + T1[2] * P1[2] + kDilation;
        const float det = a * c - b * b;
        const float id2 = 1.0f / (det * det);

        // Inverse 2x2: conic (A, B, C) = (c, -b, a) / det.
        const float ga = (-c * c * gco.x + b * c * gco.y - b * b * gco.z) * id2;
        const float gb = (2.f * b * c * gco.x - (a * c + b * b) * gco.y + 2.f * a * b * gco.z) * id2;
        const float gc = (-b * b * gco.x + a * b * gco.y - a * a * gco.z) * id2;
        gop = gco.w;

        // Sigma_2d = T Sigma T^T: gradients to T's rows and to Sigma.
        float gT0[3], gT1[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            gT0[j] = 2.f * ga * P0[j] + gb * P1[j];
            gT1[j] = gb * P0[j] + 2.f * gc * P1[j];
        }
        // T = J W: gradients to the four non-zero entries of J.
        const float gJ00 = gT0[0] * W[0] + gT0[1] * W[1] + gT0[2] * W[2];
        const float gJ02 = gT0[0] * W[6] + gT0[1] * W[7] + gT0[2] * W[8];
        const float gJ11 = gT1[0] * W[3] + gT1[1] * W[4] + gT1[2] * W[5];
        const float gJ12 = gT1[0] * W[6] + gT1[1] * W[7] + gT1[2] * W[8];

        // Pinhole and J as functions of the camera-space centre.
        float gpx = guv.x * fx * iz;
        float gpy = guv.y * fy * iz;
        float gpz = -(guv.x * fx * px + guv.y * fy * py) * iz2 - (gJ00 * fx + gJ11 * fy) * iz2;
        if (cx_on) {
            gpz += gJ02 * fx * Lx * iz2;
        } else {
            gpx -= gJ02 * fx * iz2;
            gpz += 2.f * gJ02 * fx * px * iz2 * iz;
        }
        if (cy_on) {
            gpz += gJ12 * fy * Ly * iz2;
        } else {
            gpy -= gJ12 * fy * iz2;
            gpz += 2.f * gJ12 * fy * py * iz2 * iz;
        }
        // p = W m + t.
        gm0 = W[0] * gpx + W[3] * gpy + W[6] * gpz;
        gm1 = W[1] * gpx + W[4] * gpy + W[7] * gpz;
        gm2 = W[2] * gpx + W[5] * gpy + W[8] * gpz;

        // Sigma = M M^T with dL/dSigma = ga T0^T T0 + gb sym(T0^T T1) + gc T1^T T1:
        // dL/dM = 2 (dL/dSigma) M, computed as 2 (ga T0^T (T0 M) + ...).
        float t0M[3], t1M[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            t0M[j] = T0[0] * M[0][j] + T0[1] * M[1][j] + T0[2] * M[2][j];
            t1M[j] = T1[0] * M[0][j] + T1[1] * M[1][j] + T1[2] * M[2][j];
        }
        float gR[3][3];
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const float gM = 2.f * ga * T0[i] * t0M[j] + gb * (T0[i] * t1M[j] + T1[i] * t0M[j]) +
                                 2.f * gc * T1[i] * t1M[j];
                gR[i][j] = gM * s[j];
                if (j == 0) gs0 += gM * R[i][0];
                if (j == 1) gs1 += gM * R[i][1];
                if (j == 2) gs2 += gM * R[i][2];
            }
        // R(q) of the unit quaternion.
        const float hw = 2.f * (-z * gR[0][1] + y * gR[0][2] + z * gR[1][0] - x * gR[1][2] - y * gR[2][0] +
                                x * gR[2][1]);
        const float hx = 2.f * (y * gR[0][1] + z * gR[0][2] + y * gR[1][0] - 2.f * x * gR[1][1] -
                                w * gR[1][2] + z * gR[2][0] + w * gR[2][1] - 2.f * x * gR[2][2]);
        const float hy = 2.f * (-2.f * y * gR[0][0] + x * gR[0][1] + w * gR[0][2] + x * gR[1][0] +
                                z * gR[1][2] - w * gR[2][0] + z * gR[2][1] - 2.f * y * gR[2][2]);
        const float hz = 2.f * (-2.f * z * gR[0][0] - w * gR[0][1] + x * gR[0][2] + w * gR[1][0] -
                                2.f * z * gR[1][1] + y * gR[1][2] + x * gR[2][0] + y * gR[2][1]);
        // q / |q|: drop the radial part, divide by |q|.
        const float rad = w * hw + x * hx + y * hy + z * hz;
        gq0 = (hw - w * rad) * iq;
        gq1 = (hx - x * rad) * iq;
        gq2 = (hy - y * rad) * iq;
        gq3 = (hz - z * rad) * iq;

        dc0 = gcol.x;
        dc1 = gcol.y;
        dc2 = gcol.z;
        if (sh != nullptr) {
            const float vx = mx - cam.campos[0], vy = my - cam.campos[1], vz = mz - cam.campos[2];
            const float vn = sqrtf(vx * vx + vy * vy + vz * vz);
            const float ivn = 1.0f / vn;
            dirx = vx * ivn;
            diry = vy * ivn;
            dirz = vz * ivn;
        }
    }

    // Colour: dL/dsh[k][ch] = dL/dc_ch Y_k(dir); dL/ddir = sum_k e_k grad Y_k
    // with e_k = sum_ch dL/dc_ch sh[k][ch]; then through dir = v / |v|.
    if (sh != nullptr) {
        const float x = dirx, y = diry, z = dirz;
        const float xx = x * x, yy = y * y, zz = z * z;
        float Y[16];
        Y[0] = kY0;
        Y[1] = -kY1 * y;
        Y[2] = kY1 * z;
        Y[3] = -kY1 * x;
        Y[4] = kY2a * x * y;
        Y[5] = -kY2a * y * z;
        Y[6] = kY2b * (2.f * zz - xx - yy);
        Y[7] = -kY2a * z * x;
        Y[8] = kY2c * (xx - yy);
        Y[9] = -kY3a * (3.f * xx - yy) * y;
        Y[10] = kY3b * x * y * z;
        Y[11] = -kY3c * (4.f * zz - xx - yy) * y;
        Y[12] = kY3d * z * (2.f * zz - 3.f * xx - 3.f * yy);
        Y[13] = -kY3c * x * (4.f * zz - xx - yy);
        Y[14] = kY3e * (xx - yy) * z;
        Y[15] = -kY3a * x * (xx - 3.f * yy);
        float e[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            if (k < n_coef) {
                // a culled Gaussian's colour gradient is zero
                const float s0 = visible ? shv[3 * k + 0] : 0.f;
                const float s1 = visible ? shv[3 * k + 1] : 0.f;
                const float s2 = visible ? shv[3 * k + 2] : 0.f;
                e[k] = dc0 * s0 + dc1 * s1 + dc2 * s2;
                grad_sh[(size_t)(3 * k + 0) * N + g] = dc0 * Y[k];
                grad_sh[(size_t)(3 * k + 1) * N + g] = dc1 * Y[k];
                grad_sh[(size_t)(3 * k + 2) * N + g] = dc2 * Y[k];
            } else {
                e[k] = 0.f;
            }
        }
        // gradient of sum_k e_k Y_k(x, y, z) term by term
        float dx = -kY1 * e[3], dy = -kY1 * e[1], dz = kY1 * e[2];
        dx += kY2a * y * e[4] - kY2b * 2.f * x * e[6] - kY2a * z * e[7] + kY2c * 2.f * x * e[8];
        dy += kY2a * x * e[4] - kY2a * z * e[5] - kY2b * 2.f * y * e[6] - kY2c * 2.f * y * e[8];
        dz += -kY2a * y * e[5] + kY2b * 4.f * z * e[6] - kY2a * x * e[7];
        dx += -kY3a * 6.f * x * y * e[9] + kY3b * y * z * e[10] + kY3c * 2.f * x * y * e[11] -
              kY3d * 6.f * x * z * e[12] - kY3c * (4.f * zz - 3.f * xx - yy) * e[13] +
              kY3e * 2.f * x * z * e[14] - kY3a * (3.f * xx - 3.f * yy) * e[15];
        dy += -kY3a * (3.f * xx - 3.f * yy) * e[9] + kY3b * x * z * e[10] -
              kY3c * (4.f * zz - xx - 3.f * yy) * e[11] - kY3d * 6.f * y * z * e[12] +
              kY3c * 2.f * x * y * e[13] - kY3e * 2.f * y * z * e[14] + kY3a * 6.f * x * y * e[15];
        dz += kY3b * x * y * e[10] - kY3c * 8.f * y * z * e[11] +
              kY3d * (6.f * zz - 3.f * xx - 3.f * yy) * e[12] - kY3c * 8.f * x * z * e[13] +
              kY3e * (xx - yy) * e[14];
        if (visible) {
            const float vx = mx - cam.campos[0], vy = my - cam.campos[1], vz = mz - cam.campos[2];
            const float ivn = 1.0f / sqrtf(vx * vx + vy * vy + vz * vz);
            const float rd = x * dx + y * dy + z * dz;
            gm0 += (dx - x * rd) * ivn;
            gm1 += (dy - y * rd) * ivn;
            gm2 += (dz - z * rd) * ivn;
        }
    } else {
        grad_rgb_in[g] = dc0;
        grad_rgb_in[N + g] = dc1;
        grad_rgb_in[2 * N + g] = dc2;
    }

    grad_means[g] = gm0;
    grad_means[N + g] = gm1;
    grad_means[2 * N + g] = gm2;
    grad_scales[g] = gs0;
    grad_scales[N + g] = gs1;
    grad_scales[2 * N + g] = gs2;
    grad_quats[g] = gq0;
    grad_quats[N + g] = gq1;
    grad_quats[2 * N + g] = gq2;
    grad_quats[3 * N + g] = gq3;
    grad_opacity[g] = gop;
}

}  // namespace

hipError_t launch_preprocess_bwd(const gs_camera& cam, int n, const float* means, const float* scales,
                                 const float* quats, const float* sh, int sh_degree,
                                 const uint32_t* tiles_touched, const float2* grad_mean2d,
                                 const float4* grad_conic_op, const float4* grad_rgb, float* grad_means,
                                 float* grad_scales, float* grad_quats, float* grad_opacity,
                                 float* grad_sh, float* grad_rgb_in, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const int n_coef = sh ? (sh_degree + 1) * (sh_degree + 1) : 0;
    hipLaunchKernelGGL(k_preprocess_bwd, dim3((n + 255) / 256), dim3(256), 0, stream, cam, n, means,
                       scales, quats, sh, n_coef, tiles_touched, grad_mean2d, grad_conic_op, grad_rgb,
                       grad_means, grad_scales, grad_quats, grad_opacity, grad_sh, grad_rgb_in);
    return hipGetLastError();
}

}  // namespace gs
