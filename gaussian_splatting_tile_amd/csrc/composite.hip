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
// n_contrib with the colour behind carried along, T_i = T_{i+1}/(1-a_i))
// and "Deliberate differences" (no gradient through a saturated alpha).
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
//  * Workgroup ids are remapped so each XCD renders a contiguous band of
//    tiles (neighbouring tiles share splats; L2 is per XCD).
//  * Backward: per splat, each wave sums its 64 pixels' nine gradient terms
//    with cross-lane adds (skipped when no lane contributed), the four
//    waves combine in LDS, and one global atomic per value per tile entry
//    lands in the per-Gaussian gradient.
#include "gs_internal.h"

namespace gs {
namespace {

constexpr int kBatch = 256;
constexpr float kLog2e = 1.4426950408889634f;

// Gaussian weight and alpha of a splat with conic (A, B, C) and opacity o at
// offset (dx, dy) from its centre:
//   power = -0.5 (A dx^2 + C dy^2) - B dx dy,  G = exp(power),
//   alpha = min(0.99, o G).
__device__ __forceinline__ void splat_alpha(float A, float B, float C, float o, float dx, float dy,
                                            float& G, float& alpha) {
    const float power = -0.5f * ((A * dx) * dx + (C * dy) * dy) - (B * dx) * dy;
    G = __builtin_amdgcn_exp2f(power * kLog2e);
    alpha = fminf(kAlphaMax, o * G);
    if (fabsf(alpha - kAlphaMin) <= kAlphaMin * 4e-6f) {
        G = (float)exp((double)power);
        alpha = fminf(kAlphaMax, o * G);
    }
}

__global__ __launch_bounds__(256) void k_composite_fwd(
    const int W, const int H, const int TX, const uint32_t* __restrict__ ranges,
    const uint32_t* __restrict__ point_list, const float4* __restrict__ xy_depth,
    const float4* __restrict__ conic_op, const float4* __restrict__ rgb, const float3 bg,
    float* __restrict__ image, float* __restrict__ final_T, uint32_t* __restrict__ n_contrib,
    uint32_t* __restrict__ n_examined) {
    __shared__ float4 s_conic[kBatch];  // A, B, C, opacity
    __shared__ float4 s_xyc[kBatch];    // u, v, r, g
    __shared__ float s_blue[kBatch];

    const int tile = xcd_contiguous(blockIdx.x, gridDim.x);
    const int tid = threadIdx.x;
    const int tx = tile % TX, ty = tile / TX;
    const int px = tx * kTile + (tid & 15);
    const int py = ty * kTile + (tid >> 4);
    const bool inside = px < W && py < H;
    const float fx = (float)px, fy = (float)py;
    const uint32_t start = ranges[2 * tile], end = ranges[2 * tile + 1];

    float T = 1.0f, C0 = 0.0f, C1 = 0.0f, C2 = 0.0f;
    uint32_t last = 0, examined = 0;
    bool done = !inside;

    for (uint32_t base = start; base < end; base += kBatch) {
        if (__syncthreads_count(done) == 256) break;
        const uint32_t j = base + tid;
        if (j < end) {
            const uint32_t g = point_list[j];
            const float4 xy = xy_depth[g];
            const float4 co = conic_op[g];
            const float4 c = rgb[g];
            s_conic[tid] = co;
            s_xyc[tid] = make_float4(xy.x, xy.y, c.x, c.y);
            s_blue[tid] = c.z;
        }
        __syncthreads();
        if (!done) {
            const int cnt = (int)min((uint32_t)kBatch, end - base);
            const uint32_t pos0 = base - start;
            for (int k = 0; k < cnt; ++k) {
                const float4 co = s_conic[k];
                const float4 xc = s_xyc[k];
                float G, alpha;
                splat_alpha(co.x, co.y, co.z, co.w, fx - xc.x, fy - xc.y, G, alpha);
                examined = pos0 + k + 1;
                if (alpha < kAlphaMin) continue;
                const float w = alpha * T;
                C0 = __builtin_fmaf(xc.z, w, C0);
                C1 = __builtin_fmaf(xc.w, w, C1);
                C2 = __builtin_fmaf(s_blue[k], w, C2);
                T = T * (1.0f - alpha);
                last = pos0 + k + 1;
                if (T < kTStop) {
                    done = true;
                    break;
                }
            }
        }
    }

    if (inside) {
        const size_t p = (size_t)py * W + px;
        const size_t plane = (size_t)W * H;
        image[p] = __builtin_fmaf(T, bg.x, C0);
        image[plane + p] = __builtin_fmaf(T, bg.y, C1);
        image[2 * plane + p] = __builtin_fmaf(T, bg.z, C2);
        final_T[p] = T;
        n_contrib[p] = last;
        if (n_examined) n_examined[p] = examined;
    }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

__global__ void k_zero(float* __restrict__ p, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

__global__ __launch_bounds__(256) void k_composite_bwd(
    const int W, const int H, const int TX, const uint32_t* __restrict__ ranges,
    const uint32_t* __restrict__ point_list, const float4* __restrict__ xy_depth,
    const float4* __restrict__ conic_op, const float4* __restrict__ rgb, const float3 bg,
    const float* __restrict__ final_T, const uint32_t* __restrict__ n_contrib,
    const float* __restrict__ dL_dimage, float* __restrict__ grad_mean2d,
    float* __restrict__ grad_conic_op, float* __restrict__ grad_rgb) {
    __shared__ float4 s_conic[kBatch];  // A, B, C, opacity
    __shared__ float4 s_xyc[kBatch];    // u, v, r, g
    __shared__ float s_blue[kBatch];
    __shared__ uint32_t s_gid[kBatch];
    __shared__ float s_grad[kBatch][9];
    __shared__ uint32_t s_maxnc;

    const int tile = xcd_contiguous(blockIdx.x, gridDim.x);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int tx = tile % TX, ty = tile / TX;
    const int px = tx * kTile + (tid & 15);
    const int py = ty * kTile + (tid >> 4);
    const bool inside = px < W && py < H;
    const float fx = (float)px, fy = (float)py;
    const uint32_t start = ranges[2 * tile], len = ranges[2 * tile + 1] - start;

    float T = 1.0f, g0 = 0.0f, g1 = 0.0f, g2 = 0.0f;
    uint32_t nc = 0;
    if (inside) {
        const size_t p = (size_t)py * W + px;
        const size_t plane = (size_t)W * H;
        T = final_T[p];
        nc = min(n_contrib[p], len);  // never walk past the tile's list
        g0 = dL_dimage[p];
        g1 = dL_dimage[plane + p];
        g2 = dL_dimage[2 * plane + p];
    }
    float B0 = bg.x, B1 = bg.y, B2 = bg.z;

    if (tid == 0) s_maxnc = 0;
    __syncthreads();
    if (nc > 0) atomicMax(&s_maxnc, nc);
    __syncthreads();
    const int maxnc = (int)s_maxnc;

    for (int bend = maxnc; bend > 0; bend -= kBatch) {
        const int bstart = bend > kBatch ? bend - kBatch : 0;
        const int cnt = bend - bstart;
        __syncthreads();  // the previous batch is fully consumed
        if (tid < cnt) {
            const uint32_t g = point_list[start + bstart + tid];
            const float4 xy = xy_depth[g];
            const float4 co = conic_op[g];
            const float4 c = rgb[g];
            s_conic[tid] = co;
            s_xyc[tid] = make_float4(xy.x, xy.y, c.x, c.y);
            s_blue[tid] = c.z;
            s_gid[tid] = g;
#pragma unroll
            for (int v = 0; v < 9; ++v) s_grad[tid][v] = 0.0f;
        }
        __syncthreads();

        for (int k = cnt - 1; k >= 0; --k) {
            float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f, d4 = 0.f, d5 = 0.f, d6 = 0.f, d7 = 0.f, d8 = 0.f;
            bool any = false;
            if (bstart + k < (int)nc) {
                const float4 co = s_conic[k];
                const float4 xc = s_xyc[k];
                const float dx = fx - xc.x, dy = fy - xc.y;
                float G, alpha;
                splat_alpha(co.x, co.y, co.z, co.w, dx, dy, G, alpha);
                if (alpha >= kAlphaMin) {
                    const float cb = s_blue[k];
                    const float Tj = T / (1.0f - alpha);
                    const float w = alpha * Tj;
                    d6 = w * g0;
                    d7 = w * g1;
                    d8 = w * g2;
                    const float dL_da = ((g0 * (xc.z - B0) + g1 * (xc.w - B1)) + g2 * (cb - B2)) * Tj;
                    const float om = 1.0f - alpha;
                    B0 = alpha * xc.z + om * B0;
                    B1 = alpha * xc.w + om * B1;
                    B2 = alpha * cb + om * B2;
                    T = Tj;
                    if (co.w * G <= kAlphaMax) {  // not saturated
                        const float dp = alpha * dL_da;
                        d5 = G * dL_da;
                        d2 = -0.5f * dx * dx * dp;
                        d3 = -dx * dy * dp;
                        d4 = -0.5f * dy * dy * dp;
                        d0 = (co.x * dx + co.y * dy) * dp;
                        d1 = (co.y * dx + co.z * dy) * dp;
                    }
                    any = true;
                }
            }
            if (__ballot(any) != 0ull) {
                d0 = wave_sum(d0); d1 = wave_sum(d1); d2 = wave_sum(d2);
                d3 = wave_sum(d3); d4 = wave_sum(d4); d5 = wave_sum(d5);
                d6 = wave_sum(d6); d7 = wave_sum(d7); d8 = wave_sum(d8);
                if (lane == 0) {
                    atomicAdd(&s_grad[k][0], d0); atomicAdd(&s_grad[k][1], d1);
                    atomicAdd(&s_grad[k][2], d2); atomicAdd(&s_grad[k][3], d3);
                    atomicAdd(&s_grad[k][4], d4); atomicAdd(&s_grad[k][5], d5);
                    atomicAdd(&s_grad[k][6], d6); atomicAdd(&s_grad[k][7], d7);
                    atomicAdd(&s_grad[k][8], d8);
                }
            }
        }
        __syncthreads();
        if (tid < cnt) {
            const uint32_t g = s_gid[tid];
            const float* sg = s_grad[tid];
            float* gm = grad_mean2d + 2 * (size_t)g;
            float* gc = grad_conic_op + 4 * (size_t)g;
            float* gr = grad_rgb + 4 * (size_t)g;
            if (sg[0] != 0.0f) unsafeAtomicAdd(gm + 0, sg[0]);
            if (sg[1] != 0.0f) unsafeAtomicAdd(gm + 1, sg[1]);
            if (sg[2] != 0.0f) unsafeAtomicAdd(gc + 0, sg[2]);
            if (sg[3] != 0.0f) unsafeAtomicAdd(gc + 1, sg[3]);
            if (sg[4] != 0.0f) unsafeAtomicAdd(gc + 2, sg[4]);
            if (sg[5] != 0.0f) unsafeAtomicAdd(gc + 3, sg[5]);
            if (sg[6] != 0.0f) unsafeAtomicAdd(gr + 0, sg[6]);
            if (sg[7] != 0.0f) unsafeAtomicAdd(gr + 1, sg[7]);
            if (sg[8] != 0.0f) unsafeAtomicAdd(gr + 2, sg[8]);
        }
    }
}

}  // namespace

hipError_t launch_composite_fwd(const gs_camera& cam, const uint32_t* ranges,
                                const uint32_t* point_list, const float4* xy_depth,
                                const float4* conic_op, const float4* rgb, float3 bg,
                                float* image, float* final_T, uint32_t* n_contrib,
                                uint32_t* n_examined, hipStream_t stream) {
    const int TX = tiles_x(cam), TY = tiles_y(cam);
    hipLaunchKernelGGL(k_composite_fwd, dim3(TX * TY), dim3(256), 0, stream, cam.width, cam.height,
                       TX, ranges, point_list, xy_depth, conic_op, rgb, bg, image, final_T,
                       n_contrib, n_examined);
    return hipGetLastError();
}

hipError_t launch_composite_bwd(const gs_camera& cam, int n, const uint32_t* ranges,
                                const uint32_t* point_list, const float4* xy_depth,
                                const float4* conic_op, const float4* rgb, float3 bg,
                                const float* final_T, const uint32_t* n_contrib,
                                const float* dL_dimage, float2* grad_mean2d,
                                float4* grad_conic_op, float4* grad_rgb, hipStream_t stream) {
    if (n > 0) {
        const size_t nm = 2 * (size_t)n, nc = 4 * (size_t)n;
        hipLaunchKernelGGL(k_zero, dim3((unsigned)((nm + 255) / 256)), dim3(256), 0, stream,
                           (float*)grad_mean2d, nm);
        hipLaunchKernelGGL(k_zero, dim3((unsigned)((nc + 255) / 256)), dim3(256), 0, stream,
                           (float*)grad_conic_op, nc);
        hipLaunchKernelGGL(k_zero, dim3((unsigned)((nc + 255) / 256)), dim3(256), 0, stream,
                           (float*)grad_rgb, nc);
    }
    const int TX = tiles_x(cam), TY = tiles_y(cam);
    hipLaunchKernelGGL(k_composite_bwd, dim3(TX * TY), dim3(256), 0, stream, cam.width, cam.height,
                       TX, ranges, point_list, xy_depth, conic_op, rgb, bg, final_T, n_contrib,
                       dL_dimage, (float*)grad_mean2d, (float*)grad_conic_op, (float*)grad_rgb);
    return hipGetLastError();
}

}  // namespace gs
