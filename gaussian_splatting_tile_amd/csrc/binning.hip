// Binning: prefix scan of the per-Gaussian tile counts, duplication into
// (tile_id << 32 | depth bits) keys, a stable LSD radix sort, tile ranges.
//
// Follows "rigel" README "Binning" (count, scan into private slices,
// expansion, the sort restricted to the bits a tile id can occupy, a range
// kernel); zenn 4.1 (hierarchical exclusive scan), 4.2 (duplicate into the
// slice), 4.3 (8-bit LSD radix sort with per-workgroup histograms, bin
// scan, per-workgroup bin offsets, in-bin rank from the flag bits set
// before a lane, ping-pong buffers), 4.4 (range boundaries, empty tiles
// cleared); learn-gs build_tile_lists (span order, ty outer, tx inner).
//
// MI355X design:
//  * The scan is reduce / scan-of-block-sums / rescan into per-Gaussian
//    offsets. The duplication is entry-parallel: each workgroup takes 2048
//    consecutive entries, finds the Gaussians that own them, stages their
//    offsets in LDS and gives every lane one entry (owner by binary search),
//    so the work is balanced however many tiles a Gaussian covers, and the
//    key and value stores are fully coalesced.
//  * The sort's in-workgroup rank uses 64-lane ballots: eight ballots, one
//    per digit bit, give every lane the mask of lanes holding its digit;
//    popcount below the lane is its rank (the zenn flag-bit rank, done on
//    wave64 without a match instruction). Per-wave digit counters in LDS
//    carry the rank across iterations, so the order stays stable.
//  * Each workgroup stages its sorted tile in LDS and writes it back as
//    contiguous runs per digit, so global writes coalesce.
//  * No inter-workgroup waiting anywhere: every kernel ends on its own.
#include "gs_internal.h"

namespace gs {
namespace {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 8;
constexpr int kScanTile = kScanThreads * kScanItems;  // Gaussians per workgroup

constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kSortItems = 8;                         // keys per lane
constexpr int kSortTile = kSortThreads * kSortItems;  // keys per workgroup
constexpr int kRadix = 256;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Inclusive scan of one value per thread across a 256-thread workgroup.
// `tmp` is LDS of 256 words. Returns the inclusive prefix; *total = sum.
template <typename T>
__device__ T block_inclusive_scan_256(T x, T* tmp, T* total) {
    const int tid = threadIdx.x;
    tmp[tid] = x;
    __syncthreads();
#pragma unroll
    for (int off = 1; off < 256; off <<= 1) {
        T y = (tid >= off) ? tmp[tid - off] : T(0);
        __syncthreads();
        x += y;
        tmp[tid] = x;
        __syncthreads();
    }
    *total = tmp[255];
    __syncthreads();
    return x;
}

// ---- scan ----

__global__ __launch_bounds__(kScanThreads) void k_scan_reduce(const uint32_t* __restrict__ counts,
                                                              int n, uint32_t* __restrict__ block_sums) {
    __shared__ uint32_t s_red[kScanThreads / 64];
    const int base = blockIdx.x * kScanTile;
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const int g = base + i * kScanThreads + threadIdx.x;
        if (g < n) sum += counts[g];
    }
    // wave reduce then across the 4 waves
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = sum;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < kScanThreads / 64; ++w) t += s_red[w];
        block_sums[blockIdx.x] = t;
    }
}

// One workgroup of 1024 threads scans up to 8192 block sums (n <= 2^24).
__global__ __launch_bounds__(1024) void k_scan_block_sums(const uint32_t* __restrict__ block_sums,
                                                          int nb, uint64_t* __restrict__ block_offsets,
                                                          uint64_t* __restrict__ total) {
    __shared__ uint64_t s[1024];
    constexpr int kPer = 8;
    const int tid = threadIdx.x;
    uint64_t local[kPer];
    uint64_t sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int idx = tid * kPer + i;
        local[i] = idx < nb ? (uint64_t)block_sums[idx] : 0;
        sum += local[i];
    }
    s[tid] = sum;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        uint64_t y = tid >= off ? s[tid - off] : 0;
        __syncthreads();
        sum += y;
        s[tid] = sum;
        __syncthreads();
    }
    uint64_t run = sum - [&] {
        uint64_t t = 0;
        for (int i = 0; i < kPer; ++i) t += local[i];
        return t;
    }();
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int idx = tid * kPer + i;
        if (idx < nb) block_offsets[idx] = run;
        run += local[i];
    }
    if (tid == 1023) *total = sum;
}

// Rescan each workgroup's 2048 counts with its global offset: offsets[g]
// is the first entry of Gaussian g.
__global__ __launch_bounds__(kScanThreads) void k_scan_offsets(const uint32_t* __restrict__ counts, int n,
                                                               const uint64_t* __restrict__ block_offsets,
                                                               uint32_t* __restrict__ offsets) {
    __shared__ uint32_t s_c[kScanTile];
    __shared__ uint32_t s_tmp[kScanThreads];
    const int tid = threadIdx.x;
    const int base = blockIdx.x * kScanTile;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const int idx = i * kScanThreads + tid;
        const int g = base + idx;
        s_c[idx] = g < n ? counts[g] : 0u;
    }
    __syncthreads();
    uint32_t c[kScanItems];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        c[i] = s_c[tid * kScanItems + i];
        sum += c[i];
    }
    uint32_t total;
    const uint32_t incl = block_inclusive_scan_256<uint32_t>(sum, s_tmp, &total);
    uint32_t run = (uint32_t)block_offsets[blockIdx.x] + (incl - sum);
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        s_c[tid * kScanItems + i] = run;
        run += c[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const int idx = i * kScanThreads + tid;
        if (base + idx < n) offsets[base + idx] = s_c[idx];
    }
}

// Last index g in [lo, hi] with offsets[g] <= e (offsets is nondecreasing;
// the answer is the Gaussian owning entry e, never a zero-count one).
__device__ __forceinline__ int owner_search(const uint32_t* __restrict__ offsets, int lo, int hi, uint32_t e) {
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offsets[mid] <= e) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Duplication, one entry per lane: entry e of Gaussian g (its k-th tile,
// k = e - offsets[g]) is the tile (x0 + k % w, y0 + k / w) of g's span.
// Each workgroup covers 2048 consecutive entries; it finds the range of
// Gaussians owning them, stages their offsets in LDS, and searches there.
constexpr int kDupThreads = 256;
constexpr int kDupItems = 8;
constexpr int kDupTile = kDupThreads * kDupItems;
constexpr int kDupWindow = 2048;  // staged offsets; longer owner ranges search global memory

__global__ __launch_bounds__(kDupThreads) void k_duplicate(
    const float4* __restrict__ xy_depth, const uint32_t* __restrict__ offsets, int n, uint32_t n_entries,
    int TX, int TY, uint64_t* __restrict__ keys, uint32_t* __restrict__ values) {
    __shared__ uint32_t s_off[kDupWindow];
    __shared__ int s_range[2];
    const int tid = threadIdx.x;
    const uint32_t e0 = blockIdx.x * kDupTile;
    const uint32_t e1 = min(e0 + (uint32_t)kDupTile, n_entries);
    if (tid < 2) s_range[tid] = owner_search(offsets, 0, n - 1, tid == 0 ? e0 : e1 - 1);
    __syncthreads();
    const int g_lo = s_range[0], g_hi = s_range[1];
    const int span = g_hi - g_lo + 1;
    const bool staged = span <= kDupWindow;
    if (staged)
        for (int i = tid; i < span; i += kDupThreads) s_off[i] = offsets[g_lo + i];
    __syncthreads();
#pragma unroll 2
    for (int it = 0; it < kDupItems; ++it) {
        const uint32_t e = e0 + it * kDupThreads + tid;
        if (e >= e1) break;
        int g;
        uint32_t off;
        if (staged) {
            int lo = 0, hi = span - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (s_off[mid] <= e) lo = mid; else hi = mid - 1;
            }
            g = g_lo + lo;
            off = s_off[lo];
        } else {
            g = owner_search(offsets, g_lo, g_hi, e);
            off = offsets[g];
        }
        const uint32_t k = e - off;
        const float4 rec = xy_depth[g];
        const Span sp = tile_span(rec.x, rec.y, rec.w, TX, TY);
        const uint32_t w = (uint32_t)(sp.x1 - sp.x0);
        // k / w and k % w: float quotient (k < 2^21) fixed up by one step
        uint32_t q = (uint32_t)((float)k * __builtin_amdgcn_rcpf((float)w));
        int r = (int)k - (int)(q * w);
        if (r < 0) { --q; r += (int)w; }
        if (r >= (int)w) { ++q; r -= (int)w; }
        const uint32_t tx = (uint32_t)sp.x0 + (uint32_t)r;
        const uint32_t ty = (uint32_t)sp.y0 + q;
        keys[e] = ((uint64_t)(ty * (uint32_t)TX + tx) << 32) | (uint64_t)__float_as_uint(rec.z);
        values[e] = (uint32_t)g;
    }
}

// ---- radix sort ----

__device__ __forceinline__ uint32_t digit_of(uint64_t key, int shift) {
    return (uint32_t)(key >> shift) & (kRadix - 1);
}

// Mask of the lanes of this wave that hold the same 8-bit digit (only valid
// lanes take part).
__device__ __forceinline__ uint64_t match_digit(uint32_t d, bool valid) {
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const bool bit = (d >> b) & 1u;
        const uint64_t m = __ballot(bit);
        peers &= bit ? m : ~m;
    }
    return valid ? peers : 0ull;
}

// Per-workgroup digit counts: counts[d * nblk + blk].
__global__ __launch_bounds__(kSortThreads) void k_digit_count(const uint64_t* __restrict__ keys,
                                                              uint32_t n, int shift, int nblk,
                                                              uint32_t* __restrict__ counts) {
    __shared__ uint32_t s_hist[kRadix];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    s_hist[tid] = 0;
    __syncthreads();
    const uint32_t base = blockIdx.x * kSortTile;
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const uint32_t pos = base + i * kSortThreads + tid;
        const bool valid = pos < n;
        const uint32_t d = valid ? digit_of(keys[pos], shift) : 0u;
        const uint64_t peers = match_digit(d, valid);
        if (valid && lane == __ffsll((unsigned long long)peers) - 1)
            atomicAdd(&s_hist[d], (uint32_t)__popcll(peers));
    }
    __syncthreads();
    counts[(size_t)tid * nblk + blockIdx.x] = s_hist[tid];
}

// Row d of counts -> exclusive prefix over workgroups (in place);
// digit_totals[d] = row sum. One workgroup per digit.
__global__ __launch_bounds__(256) void k_digit_scan(uint32_t* __restrict__ counts, int nblk,
                                                    uint32_t* __restrict__ digit_totals) {
    __shared__ uint32_t s_tmp[256];
    uint32_t* row = counts + (size_t)blockIdx.x * nblk;
    uint32_t carry = 0;
    for (int base = 0; base < nblk; base += 256) {
        const int i = base + threadIdx.x;
        const uint32_t x = i < nblk ? row[i] : 0u;
        uint32_t tot;
        const uint32_t incl = block_inclusive_scan_256<uint32_t>(x, s_tmp, &tot);
        if (i < nblk) row[i] = carry + incl - x;
        carry += tot;
    }
    if (threadIdx.x == 0) digit_totals[blockIdx.x] = carry;
}

// Stable scatter of one 2048-key tile. Wave w ranks the keys at
// [tile + w * 512, +512) in 8 rounds of 64 consecutive keys; the rank of a
// key among equal digits is (keys of that digit in earlier rounds of this
// wave) + (lanes below it in its round holding the digit). Waves are then
// ordered by index, workgroups by the per-digit offsets.
__global__ __launch_bounds__(kSortThreads) void k_scatter(
    const uint64_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in, uint32_t n,
    int shift, int nblk, const uint32_t* __restrict__ counts, const uint32_t* __restrict__ digit_totals,
    uint64_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out) {
    __shared__ uint32_t s_wcount[kSortWaves][kRadix];  // per-wave digit counts
    __shared__ uint32_t s_local_start[kRadix];         // digit start in the staged tile
    __shared__ uint32_t s_global[kRadix];              // digit start in the output
    __shared__ uint32_t s_tmp[256];
    __shared__ uint64_t s_keys[kSortTile];
    __shared__ uint32_t s_vals[kSortTile];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const uint32_t base = blockIdx.x * kSortTile;

#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) s_wcount[w][tid] = 0;
    __syncthreads();

    uint64_t key[kSortItems];
    uint32_t val[kSortItems];
    uint32_t rank[kSortItems];
    const uint32_t seg = base + wave * (64 * kSortItems);
#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const uint32_t pos = seg + i * 64 + lane;
        const bool valid = pos < n;
        key[i] = valid ? keys_in[pos] : ~0ull;
        val[i] = valid ? vals_in[pos] : 0u;
        const uint32_t d = digit_of(key[i], shift);
        const uint64_t peers = match_digit(d, valid);
        const uint64_t below = peers & ((1ull << lane) - 1ull);
        uint32_t before = 0;
        if (valid) before = s_wcount[wave][d];
        rank[i] = before + (uint32_t)__popcll(below);
        if (valid && below == 0ull) s_wcount[wave][d] = before + (uint32_t)__popcll(peers);
    }
    __syncthreads();

    // digit d = tid: exclusive prefix over waves, tile-local start, global start
    {
        const int d = tid;
        uint32_t acc = 0;
#pragma unroll
        for (int w = 0; w < kSortWaves; ++w) {
            const uint32_t c = s_wcount[w][d];
            s_wcount[w][d] = acc;
            acc += c;
        }
        uint32_t tot;
        const uint32_t incl = block_inclusive_scan_256<uint32_t>(acc, s_tmp, &tot);
        s_local_start[d] = incl - acc;
        const uint32_t gt = digit_totals[d];
        uint32_t tot2;
        const uint32_t gincl = block_inclusive_scan_256<uint32_t>(gt, s_tmp, &tot2);
        s_global[d] = (gincl - gt) + counts[(size_t)d * nblk + blockIdx.x];
    }
    __syncthreads();

#pragma unroll
    for (int i = 0; i < kSortItems; ++i) {
        const uint32_t pos = seg + i * 64 + lane;
        if (pos < n) {
            const uint32_t d = digit_of(key[i], shift);
            const uint32_t slot = s_local_start[d] + s_wcount[wave][d] + rank[i];
            s_keys[slot] = key[i];
            s_vals[slot] = val[i];
        }
    }
    __syncthreads();

    const uint32_t valid_n = n - base < (uint32_t)kSortTile ? n - base : (uint32_t)kSortTile;
    for (uint32_t s = tid; s < valid_n; s += kSortThreads) {
        const uint64_t k = s_keys[s];
        const uint32_t d = digit_of(k, shift);
        const uint32_t out = s_global[d] + (s - s_local_start[d]);
        keys_out[out] = k;
        vals_out[out] = s_vals[s];
    }
}

// ---- tile ranges ----

__global__ void k_fill_u32(uint32_t* __restrict__ p, size_t n, uint32_t v) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

__global__ void k_ranges(const uint64_t* __restrict__ keys, uint32_t n, uint32_t* __restrict__ ranges) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t t = (uint32_t)(keys[i] >> 32);
    if (i == 0 || (uint32_t)(keys[i - 1] >> 32) != t) ranges[2 * (size_t)t] = i;
    if (i == n - 1 || (uint32_t)(keys[i + 1] >> 32) != t) ranges[2 * (size_t)t + 1] = i + 1;
}

}  // namespace

size_t bin_scratch_layout(int n, int64_t capacity, BinScratch* out, void* base) {
    const size_t nb_scan = (size_t)(n + kScanTile - 1) / kScanTile;
    const size_t nb_sort = (size_t)((capacity + kSortTile - 1) / kSortTile);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align256(bytes > 0 ? bytes : 1);
        return at;
    };
    const size_t o_bs = take(nb_scan * 4);
    const size_t o_bo = take(nb_scan * 8);
    const size_t o_tot = take(8);
    const size_t o_off = take((size_t)n * 4);
    const size_t o_kt = take((size_t)capacity * 8);
    const size_t o_vt = take((size_t)capacity * 4);
    const size_t o_cnt = take((size_t)kRadix * nb_sort * 4);
    const size_t o_dt = take((size_t)kRadix * 4);
    if (out && base) {
        char* b = (char*)base;
        out->block_sums = (uint32_t*)(b + o_bs);
        out->block_offsets = (uint64_t*)(b + o_bo);
        out->total = (uint64_t*)(b + o_tot);
        out->offsets = (uint32_t*)(b + o_off);
        out->keys_tmp = (uint64_t*)(b + o_kt);
        out->vals_tmp = (uint32_t*)(b + o_vt);
        out->counts = (uint32_t*)(b + o_cnt);
        out->digit_totals = (uint32_t*)(b + o_dt);
    }
    return off;
}

hipError_t launch_scan(int n, const uint32_t* tiles_touched, const BinScratch& s, hipStream_t stream) {
    const int nb = (n + kScanTile - 1) / kScanTile;
    hipLaunchKernelGGL(k_scan_reduce, dim3(nb), dim3(kScanThreads), 0, stream, tiles_touched, n,
                       s.block_sums);
    hipLaunchKernelGGL(k_scan_block_sums, dim3(1), dim3(1024), 0, stream, s.block_sums, nb,
                       s.block_offsets, s.total);
    hipLaunchKernelGGL(k_scan_offsets, dim3(nb), dim3(kScanThreads), 0, stream, tiles_touched, n,
                       s.block_offsets, s.offsets);
    return hipGetLastError();
}

hipError_t launch_duplicate(const gs_camera& cam, int n, uint32_t n_entries, const float4* xy_depth,
                            const BinScratch& s, uint64_t* keys, uint32_t* values, hipStream_t stream) {
    if (n_entries == 0) return hipSuccess;
    const unsigned blocks = (n_entries + kDupTile - 1) / kDupTile;
    hipLaunchKernelGGL(k_duplicate, dim3(blocks), dim3(kDupThreads), 0, stream, xy_depth, s.offsets, n,
                       n_entries, tiles_x(cam), tiles_y(cam), keys, values);
    return hipGetLastError();
}

int radix_pass_count(int key_bits) { return (key_bits + 7) / 8; }

bool radix_input_in_tmp(int key_bits) { return (radix_pass_count(key_bits) & 1) != 0; }

hipError_t launch_radix_sort(uint64_t* keys, uint32_t* values, uint32_t n, int key_bits,
                             const BinScratch& s, hipStream_t stream) {
    const int passes = radix_pass_count(key_bits);
    const bool in_tmp = (passes & 1) != 0;
    uint64_t* kin = in_tmp ? s.keys_tmp : keys;
    uint32_t* vin = in_tmp ? s.vals_tmp : values;
    uint64_t* kout = in_tmp ? keys : s.keys_tmp;
    uint32_t* vout = in_tmp ? values : s.vals_tmp;
    if (n <= 1) {
        if (in_tmp && n == 1) {
            hipError_t e = hipMemcpyAsync(keys, kin, 8, hipMemcpyDeviceToDevice, stream);
            if (e == hipSuccess) e = hipMemcpyAsync(values, vin, 4, hipMemcpyDeviceToDevice, stream);
            return e;
        }
        return hipSuccess;
    }
    const int nblk = (int)((n + kSortTile - 1) / kSortTile);
    for (int p = 0; p < passes; ++p) {
        const int shift = 8 * p;
        hipLaunchKernelGGL(k_digit_count, dim3(nblk), dim3(kSortThreads), 0, stream, kin, n, shift,
                           nblk, s.counts);
        hipLaunchKernelGGL(k_digit_scan, dim3(kRadix), dim3(256), 0, stream, s.counts, nblk,
                           s.digit_totals);
        hipLaunchKernelGGL(k_scatter, dim3(nblk), dim3(kSortThreads), 0, stream, kin, vin, n, shift,
                           nblk, s.counts, s.digit_totals, kout, vout);
        uint64_t* tk = kin; kin = kout; kout = tk;
        uint32_t* tv = vin; vin = vout; vout = tv;
    }
    return hipGetLastError();
}

hipError_t launch_tile_ranges(const uint64_t* keys, uint32_t n_entries, int n_tiles,
                              uint32_t* ranges, hipStream_t stream) {
    const size_t words = 2 * (size_t)n_tiles;
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                       ranges, words, 0u);
    if (n_entries > 0)
        hipLaunchKernelGGL(k_ranges, dim3((n_entries + 255) / 256), dim3(256), 0, stream, keys,
                           n_entries, ranges);
    return hipGetLastError();
}

}  // namespace gs
