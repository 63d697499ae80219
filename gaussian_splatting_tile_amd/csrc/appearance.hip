// Appearance MLP ("rigel" README, section "Appearance MLP"): per Gaussian a
// latent of L floats and the unit view direction go through H ReLU units
// and 3 sigmoid units, giving the Gaussian's colour; the backward gives the
// latents' gradients and the weights' gradients summed over all Gaussians.
// The view direction is a constant of the backward, as on that page.
//
// Weights, packed: W1 [H][L+3] (row i = hidden unit i; columns the latent,
// then the direction x, y, z), b1 [H], W2 [3][H], b2 [3]; at most 29
// latents and 64 hidden units, as on that page.
//
// MI355X design:
//  * One thread per Gaussian; the weights sit in LDS and every lane of a
//    wave reads the same weight at the same time (a broadcast, no bank
//    conflicts). Latents and colours are structure-of-arrays, so each load
//    and store is coalesced.
//  * z_i is summed in float32 in input order with separate multiply and add
//    (the library is built without contraction); the active set z_i > 0 is
//    thereby decided identically in the forward, the backward and any host
//    evaluation of the same sums.
//  * Backward: each workgroup of 128 Gaussians keeps the inputs, the
//    hidden activations and their gradients column-wise in LDS (rows padded
//    to 132 floats: 16-byte aligned and 4 banks apart) and forms its partial
//    weight gradients as dot products over its Gaussians, four independent
//    fused multiply-add chains per product read 16 bytes at a time (no
//    atomics, no contention); a second kernel sums the per-workgroup
//    partials in a fixed order. Results are deterministic.
//  * The sums z_i of four hidden units are interleaved (each still in input
//    order), so a thread keeps four independent chains in flight.
//  * The direction is computed as the preprocess computes the SH direction.
#include "gs_internal.h"

namespace gs {
namespace {

constexpr int kAppThreads = 128;
constexpr int kAppPitch = kAppThreads + 4;  // LDS row pitch (floats): 16-byte rows, 4 banks apart
constexpr int kMaxIn = GS_APP_MAX_LATENT + 3;

__device__ __forceinline__ void view_dir(const gs_camera& cam, const float* __restrict__ means, size_t N, int g,
                                         float& dx, float& dy, float& dz) {
    const float vx = means[g] - cam.campos[0], vy = means[N + g] - cam.campos[1], vz = means[2 * N + g] - cam.campos[2];
    const float vn = sqrtf((vx * vx + vy * vy) + vz * vz);
    dx = vx / vn;
    dy = vy / vn;
    dz = vz / vn;
}

// Loads the packed weights into LDS.
__device__ __forceinline__ void stage_weights(const float* __restrict__ weights, int P, float* s_w) {
    for (int p = threadIdx.x; p < P; p += blockDim.x) s_w[p] = weights[p];
}

__device__ __forceinline__ float sigmoid(float y) { return 1.0f / (1.0f + __expf(-y)); }

// z of hidden units i0 .. i0 + 3 (those below H): z_i = b1_i + W1[i][0] x_0
// + W1[i][1] x_1 + ..., each summed in input order with separate multiply
// and add; the four sums are interleaved.
__device__ __forceinline__ void hidden4(const float* W1, const float* b1, int K, int H, int i0, const float* x,
                                        float z[4]) {
    const float* w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = min(i0 + u, H - 1);  // a unit past H repeats the last one; its result is unused
        w[u] = W1 + i * K;
        z[u] = b1[i];
    }
#pragma unroll
    for (int j = 0; j < kMaxIn; ++j)
        if (j < K) {
#pragma unroll
            for (int u = 0; u < 4; ++u) z[u] = z[u] + w[u][j] * x[j];
        }
}

__global__ __launch_bounds__(kAppThreads) void k_appearance_fwd(const gs_camera cam, const int n,
                                                                const float* __restrict__ means,
                                                                const float* __restrict__ latent, const int L,
                                                                const int H, const float* __restrict__ weights,
                                                                float* __restrict__ rgb) {
    extern __shared__ float s_w[];
    const int K = L + 3;
    const int P = H * K + 4 * H + 3;
    stage_weights(weights, P, s_w);
    __syncthreads();
    const int g = blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= n) return;
    const size_t N = (size_t)n;
    const float* W1 = s_w;
    const float* b1 = W1 + H * K;
    const float* W2 = b1 + H;
    const float* b2 = W2 + 3 * H;

    float x[kMaxIn];
#pragma unroll
    for (int j = 0; j < kMaxIn; ++j) x[j] = j < L ? latent[(size_t)j * N + g] : 0.0f;
    float d0, d1, d2;
    view_dir(cam, means, N, g, d0, d1, d2);
#pragma unroll
    for (int j = 0; j < kMaxIn; ++j) {
        if (j == L) x[j] = d0;
        if (j == L + 1) x[j] = d1;
        if (j == L + 2) x[j] = d2;
    }
    float y0 = b2[0], y1 = b2[1], y2 = b2[2];
    for (int i0 = 0; i0 < H; i0 += 4) {
        float z[4];
        hidden4(W1, b1, K, H, i0, x, z);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u;
            if (i < H) {
                const float h = z[u] > 0.0f ? z[u] : 0.0f;
                y0 = __builtin_fmaf(W2[i], h, y0);
                y1 = __builtin_fmaf(W2[H + i], h, y1);
                y2 = __builtin_fmaf(W2[2 * H + i], h, y2);
            }
        }
    }
    rgb[g] = sigmoid(y0);
    rgb[N + g] = sigmoid(y1);
    rgb[2 * N + g] = sigmoid(y2);
}

// Per-Gaussian backward plus the workgroup's partial weight gradients
// (partials [P][gridDim.x]: each weight's partials contiguous).
__global__ __launch_bounds__(kAppThreads) void k_appearance_bwd(
    const gs_camera cam, const int n, const float* __restrict__ means, const float* __restrict__ latent,
    const int L, const int H, const float* __restrict__ weights, const float* __restrict__ grad_rgb,
    float* __restrict__ grad_latent, float* __restrict__ partials) {
    extern __shared__ float s_mem[];
    const int K = L + 3;
    const int P = H * K + 4 * H + 3;
    float* s_w = s_mem;                          // [P]
    float* s_x = s_w + ((P + 3) & ~3);           // [K][pitch]    inputs
    float* s_h = s_x + K * kAppPitch;            // [H][pitch]    hidden activations
    float* s_dz = s_h + H * kAppPitch;           // [H][pitch]    gradients at the ReLU inputs
    float* s_dy = s_dz + H * kAppPitch;          // [3][pitch]    gradients at the sigmoid inputs
    stage_weights(weights, P, s_w);
    __syncthreads();
    const float* W1 = s_w;
    const float* b1 = W1 + H * K;
    const float* W2 = b1 + H;
    const float* b2 = W2 + 3 * H;
    const int t = threadIdx.x;
    const int g = blockIdx.x * blockDim.x + t;
    const bool valid = g < n;
    const size_t N = (size_t)n;

    if (valid) {
        float x[kMaxIn];
#pragma unroll
        for (int j = 0; j < kMaxIn; ++j) x[j] = j < L ? latent[(size_t)j * N + g] : 0.0f;
        float d0, d1, d2;
        view_dir(cam, means, N, g, d0, d1, d2);
#pragma unroll
        for (int j = 0; j < kMaxIn; ++j) {
            if (j == L) x[j] = d0;
            if (j == L + 1) x[j] = d1;
            if (j == L + 2) x[j] = d2;
            if (j < K) s_x[j * kAppPitch + t] = x[j];
        }
        // forward again, keeping the activations
        float y0 = b2[0], y1 = b2[1], y2 = b2[2];
        for (int i0 = 0; i0 < H; i0 += 4) {
            float z[4];
            hidden4(W1, b1, K, H, i0, x, z);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u;
                if (i < H) {
                    const float h = z[u] > 0.0f ? z[u] : 0.0f;
                    s_h[i * kAppPitch + t] = h;
                    // the active set: dz is kept only where z > 0
                    s_dz[i * kAppPitch + t] = z[u] > 0.0f ? 1.0f : 0.0f;
                    y0 = __builtin_fmaf(W2[i], h, y0);
                    y1 = __builtin_fmaf(W2[H + i], h, y1);
                    y2 = __builtin_fmaf(W2[2 * H + i], h, y2);
                }
            }
        }
        // through the sigmoid: dy = g s (1 - s)
        const float s0 = sigmoid(y0), s1 = sigmoid(y1), s2 = sigmoid(y2);
        const float e0 = grad_rgb[g] * s0 * (1.0f - s0);
        const float e1 = grad_rgb[N + g] * s1 * (1.0f - s1);
        const float e2 = grad_rgb[2 * N + g] * s2 * (1.0f - s2);
        s_dy[t] = e0;
        s_dy[kAppPitch + t] = e1;
        s_dy[2 * kAppPitch + t] = e2;
        // through the hidden layer, and to the latents
        float gl[kMaxIn];
#pragma unroll
        for (int j = 0; j < kMaxIn; ++j) gl[j] = 0.0f;
        for (int i = 0; i < H; ++i) {
            const float dh = W2[i] * e0 + W2[H + i] * e1 + W2[2 * H + i] * e2;
            const float dz = s_dz[i * kAppPitch + t] * dh;
            s_dz[i * kAppPitch + t] = dz;
            const float* w = W1 + i * K;
#pragma unroll
            for (int j = 0; j < kMaxIn; ++j)
                if (j < L) gl[j] += w[j] * dz;
        }
#pragma unroll
        for (int j = 0; j < kMaxIn; ++j)
            if (j < L) grad_latent[(size_t)j * N + g] = gl[j];
    } else {
        // idle slots contribute nothing to the partial sums
        for (int j = 0; j < K; ++j) s_x[j * kAppPitch + t] = 0.0f;
        for (int i = 0; i < H; ++i) {
            s_h[i * kAppPitch + t] = 0.0f;
            s_dz[i * kAppPitch + t] = 0.0f;
        }
        for (int c = 0; c < 3; ++c) s_dy[c * kAppPitch + t] = 0.0f;
    }
    __syncthreads();

    // partial weight gradients of this workgroup: one dot product over its
    // Gaussians per weight, in slot order
    float* out = partials + blockIdx.x;
    for (int p = t; p < P; p += kAppThreads) {
        const float* a;
        const float* b = nullptr;
        if (p < H * K) {                 // dW1[i][j] = sum dz_i x_j
            a = s_dz + (p / K) * kAppPitch;
            b = s_x + (p % K) * kAppPitch;
        } else if (p < H * K + H) {      // db1[i] = sum dz_i
            a = s_dz + (p - H * K) * kAppPitch;
        } else if (p < H * K + 4 * H) {  // dW2[c][i] = sum dy_c h_i
            const int q = p - H * K - H;
            a = s_dy + (q / H) * kAppPitch;
            b = s_h + (q % H) * kAppPitch;
        } else {                         // db2[c] = sum dy_c
            a = s_dy + (p - H * K - 4 * H) * kAppPitch;
        }
        const float4* a4 = reinterpret_cast<const float4*>(a);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        if (b) {
            const float4* b4 = reinterpret_cast<const float4*>(b);
#pragma unroll 8
            for (int s = 0; s < kAppThreads / 4; ++s) {
                const float4 u = a4[s], v = b4[s];
                acc.x = __builtin_fmaf(u.x, v.x, acc.x);
                acc.y = __builtin_fmaf(u.y, v.y, acc.y);
                acc.z = __builtin_fmaf(u.z, v.z, acc.z);
                acc.w = __builtin_fmaf(u.w, v.w, acc.w);
            }
        } else {
#pragma unroll 8
            for (int s = 0; s < kAppThreads / 4; ++s) {
                const float4 u = a4[s];
                acc.x += u.x;
                acc.y += u.y;
                acc.z += u.z;
                acc.w += u.w;
            }
        }
        out[(size_t)p * gridDim.x] = (acc.x + acc.y) + (acc.z + acc.w);
    }
}

// grad_weights[p] = sum over workgroups b of partials[p][b], b in order:
// one workgroup per weight, a strided sum per thread, then a fixed tree.
__global__ __launch_bounds__(256) void k_appearance_reduce(const float* __restrict__ partials, int nblk, int P,
                                                          float* __restrict__ grad_weights) {
    __shared__ float s_sum[256];
    const int p = blockIdx.x, t = threadIdx.x;
    float acc = 0.0f;
    const float* row = partials + (size_t)p * nblk;
    for (int b = t; b < nblk; b += 256) acc += row[b];
    s_sum[t] = acc;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (t < off) s_sum[t] += s_sum[t + off];
        __syncthreads();
    }
    if (t == 0) grad_weights[p] = s_sum[0];
}

}  // namespace

int appearance_params(int L, int H) { return H * (L + 3) + 4 * H + 3; }

size_t appearance_bwd_scratch(int n, int L, int H) {
    const size_t nblk = (size_t)(n + kAppThreads - 1) / kAppThreads;
    return nblk * (size_t)appearance_params(L, H) * sizeof(float);
}

hipError_t launch_appearance_fwd(const gs_camera& cam, int n, const float* means, const float* latent, int L,
                                 int H, const float* weights, float* rgb, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    const size_t lds = (size_t)appearance_params(L, H) * sizeof(float);
    hipLaunchKernelGGL(k_appearance_fwd, dim3((n + kAppThreads - 1) / kAppThreads), dim3(kAppThreads), lds, stream,
                       cam, n, means, latent, L, H, weights, rgb);
    return hipGetLastError();
}

hipError_t launch_appearance_bwd(const gs_camera& cam, int n, const float* means, const float* latent, int L,
                                 int H, const float* weights, const float* grad_rgb, float* grad_latent,
                                 float* grad_weights, float* partials, hipStream_t stream) {
    const int P = appearance_params(L, H);
    if (n <= 0) return launch_fill_u32((uint32_t*)grad_weights, (size_t)P, 0u, stream);  // 0.0f bits
    const int nblk = (n + kAppThreads - 1) / kAppThreads;
    const int K = L + 3;
    const size_t lds = (size_t)(((P + 3) & ~3) + (K + 2 * H + 3) * kAppPitch) * sizeof(float);
    if (lds > 65536) {  // up to 93 KB at 29 latents and 64 units
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_appearance_bwd),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_appearance_bwd, dim3(nblk), dim3(kAppThreads), lds, stream, cam, n, means, latent, L, H,
                       weights, grad_rgb, grad_latent, partials);
    hipLaunchKernelGGL(k_appearance_reduce, dim3(P), dim3(256), 0, stream, (const float*)partials, nblk, P,
                       grad_weights);
    return hipGetLastError();
}

}  // namespace gs
