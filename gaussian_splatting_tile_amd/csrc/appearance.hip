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
//    and store is coalesced. (Reading the weights through the scalar cache
//    instead measured slower: each hidden unit then waits on its loads.)
//  * z_i is summed in float32 in input order with separate multiply and add
//    (the library is built without contraction); the active set z_i > 0 is
//    thereby decided identically in the forward, the backward and any host
//    evaluation of the same sums. The sums of four hidden units are
//    interleaved (each still in input order), so a thread keeps four
//    independent chains in flight.
//  * Backward: each workgroup of 128 Gaussians forms its partial weight
//    gradients as dot products over its Gaussians, four independent fused
//    multiply-add chains per product read 16 bytes at a time from
//    column-wise LDS rows (padded to 132 floats: 16-byte aligned, 4 banks
//    apart), in two phases over one LDS tile: dW2 and db2 from the hidden
//    activations and the sigmoid-input gradients, then dW1 and db1 from the
//    ReLU-input gradients and the inputs. The tile holds at most H + 32
//    rows (with the weights about 25 KB at 8 latents and 32 units, half of
//    keeping every row at once), so more workgroups share a compute unit. A
//    second kernel sums the per-workgroup partials in a fixed order (no
//    atomics; results are deterministic).
//  * The direction is computed as the preprocess computes the SH direction.
#include <algorithm>

#include "gs_internal.h"

namespace gs {
namespace {

constexpr int kAppThreads = 128;
constexpr int kAppPitch = kAppThreads + 4;  // LDS row pitch (floats): 16-byte rows, 4 banks apart

__device__ __forceinline__ void view_dir(const gs_camera& cam, const float* __restrict__ means, size_t N, int g,
                                         float& dx, float& dy, float& dz) {
    const float vx = means[g] - cam.campos[0], vy = means[N + g] - cam.campos[1], vz = means[2 * N + g] - cam.campos[2];
    const float vn = sqrtf((vx * vx + vy * vy) + vz * vz);
    dx = vx / vn;
    dy = vy / vn;
    dz = vz / vn;
}

// The weights in LDS, laid out for 16-byte reads: W1 input-major
// (w1t[j][i], units padded to a multiple of 4, so four units of one input
// are one read), W1 unit-major (w1r[i][j]), b1, W2 unit-major
// (w2t[i] = (W2[0][i], W2[1][i], W2[2][i], 0)) and b2. Inputs are padded to
// K4, a multiple of 4, in both W1 layouts; the padding is zero.
struct AppLds {
    float* w1t;
    float* w1r;
    float* b1;
    float4* w2t;
    float* b2;
    int H4, K4;
};
__host__ __device__ inline int app_lds_floats(int L, int H) {
    const int K = L + 3, H4 = (H + 3) & ~3, K4 = (K + 3) & ~3;
    return K4 * H4 + H * K4 + H4 + 4 * H + 4;
}
__device__ __forceinline__ AppLds app_lds(float* base, int L, int H) {
    const int K = L + 3, H4 = (H + 3) & ~3, K4 = (K + 3) & ~3;
    AppLds w;
    w.w1t = base;
    w.w1r = w.w1t + K4 * H4;
    w.b1 = w.w1r + H * K4;
    w.w2t = reinterpret_cast<float4*>(w.b1 + H4);
    w.b2 = reinterpret_cast<float*>(w.w2t + H);
    w.H4 = H4;
    w.K4 = K4;
    return w;
}
// Loads the packed weights (W1 [H][K], b1 [H], W2 [3][H], b2 [3]) into
// those layouts; padding is zero.
__device__ __forceinline__ void stage_weights(const float* __restrict__ weights, int L, int H, float* base) {
    const int K = L + 3, H4 = (H + 3) & ~3, K4 = (K + 3) & ~3;
    const AppLds w = app_lds(base, L, H);
    for (int q = threadIdx.x; q < app_lds_floats(L, H); q += blockDim.x) base[q] = 0.0f;
    __syncthreads();
    const int P = H * K + 4 * H + 3;
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        const float v = weights[p];
        if (p < H * K) {
            const int i = p / K, j = p - i * K;
            w.w1t[j * H4 + i] = v;
            w.w1r[i * K4 + j] = v;
        } else if (p < H * K + H) {
            w.b1[p - H * K] = v;
        } else if (p < H * K + 4 * H) {
            const int q = p - H * K - H, c = q / H, i = q - c * H;
            reinterpret_cast<float*>(w.w2t + i)[c] = v;
        } else {
            w.b2[p - H * K - 4 * H] = v;
        }
    }
}

__device__ __forceinline__ float sigmoid(float y) { return 1.0f / (1.0f + __expf(-y)); }

// z of hidden units i0 .. i0 + 3 (i0 a multiple of 4; units past H are
// padding): z_i = b1_i + W1[i][0] x_0 + W1[i][1] x_1 + ..., each summed in
// input order with separate multiply and add; the four sums are
// interleaved, their weights of one input read as one float4.
//
// KP = K4 / 4: the inputs past K are zero with zero weights, so each adds an
// exact zero after the real terms and z is unchanged (a fixed trip count
// lets every loop unroll without per-input branches).
template <int KP>
__device__ __forceinline__ void hidden4(const AppLds& w, int i0, const float* x, float z[4]) {
    const float4 b = *reinterpret_cast<const float4*>(w.b1 + i0);
    z[0] = b.x;
    z[1] = b.y;
    z[2] = b.z;
    z[3] = b.w;
#pragma unroll
    for (int j = 0; j < 4 * KP; ++j) {
        const float4 c = *reinterpret_cast<const float4*>(w.w1t + j * w.H4 + i0);
        z[0] = z[0] + c.x * x[j];
        z[1] = z[1] + c.y * x[j];
        z[2] = z[2] + c.z * x[j];
        z[3] = z[3] + c.w * x[j];
    }
}

// The inputs of Gaussian g: its latent, then the unit view direction,
// then zeros up to 4 KP.
template <int KP>
__device__ __forceinline__ void inputs(const gs_camera& cam, const float* __restrict__ means,
                                       const float* __restrict__ latent, size_t N, int L, int g, float x[4 * KP]) {
#pragma unroll
    for (int j = 0; j < 4 * KP; ++j) x[j] = j < L ? latent[(size_t)j * N + g] : 0.0f;
    float d0, d1, d2;
    view_dir(cam, means, N, g, d0, d1, d2);
#pragma unroll
    for (int j = 0; j < 4 * KP; ++j) {
        if (j == L) x[j] = d0;
        if (j == L + 1) x[j] = d1;
        if (j == L + 2) x[j] = d2;
    }
}

template <int KP>
__global__ __launch_bounds__(kAppThreads) void k_appearance_fwd(const gs_camera cam, const int n,
                                                                const float* __restrict__ means,
                                                                const float* __restrict__ latent, const int L,
                                                                const int H, const float* __restrict__ weights,
                                                                float* __restrict__ rgb) {
    extern __shared__ float s_w[];
    stage_weights(weights, L, H, s_w);
    __syncthreads();
    const int g = blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= n) return;
    const size_t N = (size_t)n;
    const AppLds w = app_lds(s_w, L, H);
    float x[4 * KP];
    inputs<KP>(cam, means, latent, N, L, g, x);
    float y0 = w.b2[0], y1 = w.b2[1], y2 = w.b2[2];
    for (int i0 = 0; i0 < H; i0 += 4) {
        float z[4];
        hidden4<KP>(w, i0, x, z);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = i0 + u;
            if (i < H) {
                const float h = z[u] > 0.0f ? z[u] : 0.0f;
                const float4 v = w.w2t[i];
                y0 = __builtin_fmaf(v.x, h, y0);
                y1 = __builtin_fmaf(v.y, h, y1);
                y2 = __builtin_fmaf(v.z, h, y2);
            }
        }
    }
    rgb[g] = sigmoid(y0);
    rgb[N + g] = sigmoid(y1);
    rgb[2 * N + g] = sigmoid(y2);
}

// sum over the workgroup's Gaussians of a[t] b[t] (b NULL: of a[t]), from
// two LDS rows of kAppThreads floats, four chains of 16-byte reads
__device__ __forceinline__ float row_dot(const float* a, const float* b) {
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
    return (acc.x + acc.y) + (acc.z + acc.w);
}

// Slot of workgroup b among nb in the partials. Workgroups go round-robin
// over the eight XCDs (b mod 8), each with its own L2; slots are handed out
// per XCD in contiguous blocks, so the 4-byte partials that fill one cache
// line come from a single L2 instead of eight (each of which would write
// back its own copy of the partly written line). A bijection on [0, nb).
__device__ __forceinline__ int xcd_slot(int b, int nb) {
    const int x = b & 7, k = b >> 3, q = nb >> 3, r = nb & 7;
    return x * q + min(x, r) + k;
}

// Per-Gaussian backward plus the workgroup's partial weight gradients
// (partials [P][gridDim.x]: each weight's partials contiguous, in slot order).
template <int KP>
__global__ __launch_bounds__(kAppThreads) void k_appearance_bwd(
    const gs_camera cam, const int n, const float* __restrict__ means, const float* __restrict__ latent,
    const int L, const int H, const float* __restrict__ weights, const float* __restrict__ grad_rgb,
    float* __restrict__ grad_latent, float* __restrict__ partials) {
    extern __shared__ float s_mem[];
    const int K = L + 3;
    float* const s_tile = s_mem;                                     // [H + max(3, K)][kAppPitch]
    float* const s_w = s_mem + (H + (K > 3 ? K : 3)) * kAppPitch;   // the weights (AppLds)
    stage_weights(weights, L, H, s_w);
    __syncthreads();
    const AppLds w = app_lds(s_w, L, H);
    const int t = threadIdx.x;
    const int g = blockIdx.x * blockDim.x + t;
    const bool valid = g < n;
    const size_t N = (size_t)n;
    float* const out = partials + xcd_slot((int)blockIdx.x, (int)gridDim.x);  // weight p's at out[p * gridDim.x]
    const size_t ps = gridDim.x;

    // 1. forward again: hidden activations to rows [0, H), the sigmoid-input
    //    gradients dy = g s (1 - s) to rows H .. H + 2; the active set as bits
    float x[4 * KP];
    uint64_t active = 0;
    float e0 = 0.0f, e1 = 0.0f, e2 = 0.0f;
    if (valid) {
        inputs<KP>(cam, means, latent, N, L, g, x);
        float y0 = w.b2[0], y1 = w.b2[1], y2 = w.b2[2];
        for (int i0 = 0; i0 < H; i0 += 4) {
            float z[4];
            hidden4<KP>(w, i0, x, z);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u;
                if (i < H) {
                    const float h = z[u] > 0.0f ? z[u] : 0.0f;
                    active |= (z[u] > 0.0f ? 1ull : 0ull) << i;
                    s_tile[i * kAppPitch + t] = h;
                    const float4 v = w.w2t[i];
                    y0 = __builtin_fmaf(v.x, h, y0);
                    y1 = __builtin_fmaf(v.y, h, y1);
                    y2 = __builtin_fmaf(v.z, h, y2);
                }
            }
        }
        const float s0 = sigmoid(y0), s1 = sigmoid(y1), s2 = sigmoid(y2);
        e0 = grad_rgb[g] * s0 * (1.0f - s0);
        e1 = grad_rgb[N + g] * s1 * (1.0f - s1);
        e2 = grad_rgb[2 * N + g] * s2 * (1.0f - s2);
    } else {
        for (int i = 0; i < H; ++i) s_tile[i * kAppPitch + t] = 0.0f;  // idle slots add nothing
    }
    s_tile[H * kAppPitch + t] = e0;
    s_tile[(H + 1) * kAppPitch + t] = e1;
    s_tile[(H + 2) * kAppPitch + t] = e2;
    __syncthreads();
    // 2. dW2[c][i] = sum dy_c h_i, db2[c] = sum dy_c
    for (int q = t; q < 3 * H + 3; q += kAppThreads) {
        const float* dy = s_tile + (H + (q < 3 * H ? q / H : q - 3 * H)) * kAppPitch;
        out[(H * K + H + q) * ps] = row_dot(dy, q < 3 * H ? s_tile + (q % H) * kAppPitch : nullptr);
    }
    __syncthreads();
    // 3. through the hidden layer: dz = (W2^T dy) on the active units, to
    //    rows [0, H); the latents' gradients; the inputs to rows H .. H + K - 1
    if (valid) {
        // gradients of every input (those past the latents are discarded)
        float gl[4 * KP];
#pragma unroll
        for (int j = 0; j < 4 * KP; ++j) gl[j] = 0.0f;
        for (int i = 0; i < H; ++i) {
            const float4 v = w.w2t[i];
            const float dh = v.x * e0 + v.y * e1 + v.z * e2;
            const float dz = (active >> i) & 1ull ? dh : 0.0f;
            s_tile[i * kAppPitch + t] = dz;
            const float4* row = reinterpret_cast<const float4*>(w.w1r + i * w.K4);
#pragma unroll
            for (int j4 = 0; j4 < KP; ++j4) {
                const float4 c = row[j4];
                gl[4 * j4] += c.x * dz;
                gl[4 * j4 + 1] += c.y * dz;
                gl[4 * j4 + 2] += c.z * dz;
                gl[4 * j4 + 3] += c.w * dz;
            }
        }
#pragma unroll
        for (int j = 0; j < 4 * KP; ++j) {
            if (j < L) grad_latent[(size_t)j * N + g] = gl[j];
            if (j < K) s_tile[(H + j) * kAppPitch + t] = x[j];
        }
    } else {
        for (int i = 0; i < H + K; ++i) s_tile[i * kAppPitch + t] = 0.0f;
    }
    __syncthreads();
    // 4. dW1[i][j] = sum dz_i x_j, db1[i] = sum dz_i
    for (int p = t; p < H * K + H; p += kAppThreads) {
        const float* dz = s_tile + (p < H * K ? p / K : p - H * K) * kAppPitch;
        out[p * ps] = row_dot(dz, p < H * K ? s_tile + (H + p % K) * kAppPitch : nullptr);
    }
}

// grad_weights[p] = sum over the slots b of partials[p][b], in a fixed
// order: one workgroup per weight, a strided sum per thread, then a fixed
// tree.
__global__ __launch_bounds__(256) void k_appearance_reduce(const float* __restrict__ partials, int nblk,
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

// The kernels for KP = ceil((L + 3) / 4), 1 .. 8, chosen at launch.
template <int KP>
hipError_t appearance_fwd_kp(const gs_camera& cam, int n, const float* means, const float* latent, int L, int H,
                             const float* weights, float* rgb, hipStream_t stream) {
    const size_t lds = (size_t)app_lds_floats(L, H) * sizeof(float);
    hipLaunchKernelGGL(k_appearance_fwd<KP>, dim3((n + kAppThreads - 1) / kAppThreads), dim3(kAppThreads), lds,
                       stream, cam, n, means, latent, L, H, weights, rgb);
    return hipGetLastError();
}

template <int KP>
hipError_t appearance_bwd_kp(const gs_camera& cam, int n, const float* means, const float* latent, int L, int H,
                             const float* weights, const float* grad_rgb, float* grad_latent, float* grad_weights,
                             float* partials, hipStream_t stream) {
    const int P = H * (L + 3) + 4 * H + 3;
    const int nblk = (n + kAppThreads - 1) / kAppThreads;
    const int K = L + 3;
    const size_t lds = (size_t)((H + std::max(3, K)) * kAppPitch + app_lds_floats(L, H)) * sizeof(float);
    if (lds > 65536) {  // up to 68 KB at 29 latents and 64 units
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_appearance_bwd<KP>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_appearance_bwd<KP>, dim3(nblk), dim3(kAppThreads), lds, stream, cam, n, means, latent, L,
                       H, weights, grad_rgb, grad_latent, partials);
    hipLaunchKernelGGL(k_appearance_reduce, dim3(P), dim3(256), 0, stream, (const float*)partials, nblk,
                       grad_weights);
    return hipGetLastError();
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
#define GS_FWD_CALL(KP) appearance_fwd_kp<KP>(cam, n, means, latent, L, H, weights, rgb, stream)
    switch ((L + 3 + 3) / 4) {
        case 1: return GS_FWD_CALL(1);
        case 2: return GS_FWD_CALL(2);
        case 3: return GS_FWD_CALL(3);
        case 4: return GS_FWD_CALL(4);
        case 5: return GS_FWD_CALL(5);
        case 6: return GS_FWD_CALL(6);
        case 7: return GS_FWD_CALL(7);
        case 8: return GS_FWD_CALL(8);
        default: return hipErrorInvalidValue;
    }
#undef GS_FWD_CALL
}

hipError_t launch_appearance_bwd(const gs_camera& cam, int n, const float* means, const float* latent, int L,
                                 int H, const float* weights, const float* grad_rgb, float* grad_latent,
                                 float* grad_weights, float* partials, hipStream_t stream) {
    if (n <= 0) return launch_fill_u32((uint32_t*)grad_weights, (size_t)appearance_params(L, H), 0u, stream);
#define GS_BWD_CALL(KP) \
    appearance_bwd_kp<KP>(cam, n, means, latent, L, H, weights, grad_rgb, grad_latent, grad_weights, partials, stream)
    switch ((L + 3 + 3) / 4) {
        case 1: return GS_BWD_CALL(1);
        case 2: return GS_BWD_CALL(2);
        case 3: return GS_BWD_CALL(3);
        case 4: return GS_BWD_CALL(4);
        case 5: return GS_BWD_CALL(5);
        case 6: return GS_BWD_CALL(6);
        case 7: return GS_BWD_CALL(7);
        case 8: return GS_BWD_CALL(8);
        default: return hipErrorInvalidValue;
    }
#undef GS_BWD_CALL
}

}  // namespace gs
