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
//  * The sort is split in two, with the same final order as one stable sort
//    of the 64-bit keys: a stable LSD sort on the tile-id bits only (two
//    8-bit passes at 1080p), then one workgroup per tile sorting its
//    segment by the 32 depth bits in LDS. Passes over digits that every
//    element of a segment shares are skipped.
//  * The in-workgroup rank uses 64-lane ballots: eight ballots, one
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

// ---- per-tile depth sort ----
//
// After the tile-id passes, each tile's entries are contiguous and in
// Gaussian-index order. Each tile's segment is then sorted by its 32 depth
// bits with a stable 8-bit LSD radix sort (passes over a digit that every
// element shares are skipped), so the final order is (tile, depth bits,
// Gaussian index): the order of one stable sort on the whole 64-bit key.
// Segment sizes vary by orders of magnitude, so there are size classes:
//   n <= 512      one wave per tile, no barriers (four tiles per workgroup)
//   n <= 2048     a 256-lane workgroup
//   n <= 8192     a 1024-lane workgroup with a 128 KB LDS arena
//   larger        the 1024-lane workgroup, chunked through global scratch
// Each class's kernel runs over all tiles and skips the others.
constexpr int kSegWaveCap = 512;
constexpr int kSegRounds = 8;  // 64-key rounds per wave

// --- one wave per tile ---

// Orders this wave's LDS accesses across lanes at a phase boundary (the
// wave's LDS operations complete in order; this keeps the compiler from
// moving them across the boundary).
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

__global__ __launch_bounds__(256) void k_segment_sort_wave(
    const uint32_t* __restrict__ seg_ranges, int n_tiles, const uint64_t* __restrict__ keys_in,
    const uint32_t* __restrict__ vals_in, uint64_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out) {
    __shared__ uint32_t s_k[4][kSegWaveCap];
    __shared__ uint32_t s_v[4][kSegWaveCap];
    __shared__ uint32_t s_cnt[4][kRadix];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wave;
    if (t >= n_tiles) return;
    const uint32_t start = seg_ranges[2 * t], end = seg_ranges[2 * t + 1];
    const int n = (int)(end - start);
    if (n <= 0 || n > kSegWaveCap) return;
    if (n == 1) {
        if (lane == 0) {
            keys_out[start] = keys_in[start];
            vals_out[start] = vals_in[start];
        }
        return;
    }
    const uint64_t hi = keys_in[start] & 0xFFFFFFFF00000000ull;
    uint32_t* cnt = s_cnt[wave];
    const int rounds = (n + 63) / 64;
    // keys and values live in registers between passes; LDS only stages the scatter
    uint32_t key[kSegRounds], val[kSegRounds];
#pragma unroll
    for (int r = 0; r < kSegRounds; ++r) {
        const int i = r * 64 + lane;
        key[r] = (r < rounds && i < n) ? (uint32_t)keys_in[start + i] : 0u;
        val[r] = (r < rounds && i < n) ? vals_in[start + i] : 0u;
    }
    uint32_t* dk = s_k[wave];
    uint32_t* dv = s_v[wave];
    for (int p = 0; p < 4; ++p) {
        const int shift = 8 * p;
#pragma unroll
        for (int j = 0; j < 4; ++j) cnt[4 * lane + j] = 0u;
        wave_sync();
        uint32_t rank[kSegRounds];
#pragma unroll
        for (int r = 0; r < kSegRounds; ++r) {
            rank[r] = 0u;
            if (r < rounds) {
                const bool valid = r * 64 + lane < n;
                const uint32_t d = (key[r] >> shift) & (kRadix - 1);
                const uint64_t peers = match_digit(d, valid);
                const uint64_t below = peers & ((1ull << lane) - 1ull);
                uint32_t before = 0;
                if (valid) before = cnt[d];
                rank[r] = before + (uint32_t)__popcll(below);
                if (valid && below == 0ull) cnt[d] = before + (uint32_t)__popcll(peers);
            }
        }
        wave_sync();
        // digit starts: lane owns digits 4 lane .. 4 lane + 3
        const uint32_t c0 = cnt[4 * lane], c1 = cnt[4 * lane + 1], c2 = cnt[4 * lane + 2], c3 = cnt[4 * lane + 3];
        if (__ballot(c0 == (uint32_t)n || c1 == (uint32_t)n || c2 == (uint32_t)n || c3 == (uint32_t)n) != 0ull)
            continue;  // one digit holds everything: this pass is the identity
        const uint32_t local = (c0 + c1) + (c2 + c3);
        uint32_t v = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = (uint32_t)__shfl_up((int)v, off, 64);
            if (lane >= off) v += y;
        }
        const uint32_t b0 = v - local;
        cnt[4 * lane] = b0;
        cnt[4 * lane + 1] = b0 + c0;
        cnt[4 * lane + 2] = b0 + c0 + c1;
        cnt[4 * lane + 3] = b0 + c0 + c1 + c2;
        wave_sync();
#pragma unroll
        for (int r = 0; r < kSegRounds; ++r) {
            if (r < rounds && r * 64 + lane < n) {
                const uint32_t d = (key[r] >> shift) & (kRadix - 1);
                const uint32_t pos = cnt[d] + rank[r];
                dk[pos] = key[r];
                dv[pos] = val[r];
            }
        }
        wave_sync();
#pragma unroll
        for (int r = 0; r < kSegRounds; ++r) {
            const int i = r * 64 + lane;
            if (r < rounds && i < n) {
                key[r] = dk[i];
                val[r] = dv[i];
            }
        }
        wave_sync();
    }
#pragma unroll
    for (int r = 0; r < kSegRounds; ++r) {
        const int i = r * 64 + lane;
        if (r < rounds && i < n) {
            keys_out[start + i] = hi | key[r];
            vals_out[start + i] = val[r];
        }
    }
}

// --- one workgroup per tile ---

template <int NW>
struct SegShared {
    uint32_t wc[NW][kRadix];  // per-wave digit counts / prefixes
    uint32_t base[kRadix];    // digit start (+ elements already placed)
    uint32_t wsum[4];
    uint32_t flag[4];         // pass p: every element has the same digit
};

// Exclusive scan of one value per thread over threads 0..255 (all threads
// of the workgroup must call it: it contains a barrier).
__device__ __forceinline__ uint32_t block_exclusive_scan_fast(uint32_t x, uint32_t* wsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t v = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)v, off, 64);
        if (lane >= off) v += y;
    }
    if (lane == 63 && wave < 4) wsum[wave] = v;
    __syncthreads();
    uint32_t pre = 0;
    for (int w = 0; w < wave && w < 4; ++w) pre += wsum[w];
    return pre + v - x;
}

// One stable counting pass over n <= NW * 64 * kSegRounds elements,
// src -> dst. Wave w ranks the contiguous elements [w q, (w + 1) q) (q a
// multiple of 64) in rounds of 64 against its own digit counters, keeping
// keys and ranks in registers; the per-wave counts give the wave prefixes
// and the histogram. Returns false (moving nothing) when all elements share
// the digit.
template <int NW>
__device__ __forceinline__ bool seg_pass_reg(const uint32_t* sk, const uint32_t* sv, uint32_t* dk,
                                             uint32_t* dv, int n, int pass, SegShared<NW>& L) {
    constexpr int NT = NW * 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int shift = 8 * pass;
    const int q = ((n + NT - 1) / NT) * 64;
    if (tid < kRadix)
#pragma unroll
        for (int w = 0; w < NW; ++w) L.wc[w][tid] = 0;
    __syncthreads();
    uint32_t key[kSegRounds], val[kSegRounds], rank[kSegRounds];
#pragma unroll
    for (int r = 0; r < kSegRounds; ++r) {
        key[r] = 0u; val[r] = 0u; rank[r] = 0u;
        if (r * 64 < q) {
            const int i = wave * q + r * 64 + lane;
            const bool valid = i < n;
            key[r] = valid ? sk[i] : 0u;
            val[r] = valid ? sv[i] : 0u;
            const uint32_t d = (key[r] >> shift) & (kRadix - 1);
            const uint64_t peers = match_digit(d, valid);
            const uint64_t below = peers & ((1ull << lane) - 1ull);
            uint32_t before = 0;
            if (valid) before = L.wc[wave][d];
            rank[r] = before + (uint32_t)__popcll(below);
            if (valid && below == 0ull) L.wc[wave][d] = before + (uint32_t)__popcll(peers);
        }
    }
    __syncthreads();
    uint32_t acc = 0;
    if (tid < kRadix) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const uint32_t c = L.wc[w][tid];
            L.wc[w][tid] = acc;
            acc += c;
        }
        if (acc == (uint32_t)n) L.flag[pass] = 1u;
    }
    const uint32_t b = block_exclusive_scan_fast(acc, L.wsum);
    if (tid < kRadix) L.base[tid] = b;
    __syncthreads();
    if (L.flag[pass]) return false;
#pragma unroll
    for (int r = 0; r < kSegRounds; ++r) {
        const int i = wave * q + r * 64 + lane;
        if (r * 64 < q && i < n) {
            const uint32_t d = (key[r] >> shift) & (kRadix - 1);
            const uint32_t pos = L.base[d] + L.wc[wave][d] + rank[r];
            dk[pos] = key[r];
            dv[pos] = val[r];
        }
    }
    __syncthreads();
    return true;
}

// The same pass for any n, chunk by chunk (a histogram sweep gives the
// digit starts; a running count per digit carries the order across chunks).
template <int NW>
__device__ __forceinline__ bool seg_pass_chunked(const uint32_t* sk, const uint32_t* sv, uint32_t* dk,
                                                 uint32_t* dv, int n, int pass, SegShared<NW>& L) {
    constexpr int NT = NW * 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int shift = 8 * pass;
    if (tid < kRadix) L.base[tid] = 0;
    __syncthreads();
    for (int c = 0; c < n; c += NT) {
        const int i = c + tid;
        const bool valid = i < n;
        const uint32_t d = valid ? (sk[i] >> shift) & (kRadix - 1) : 0u;
        const uint64_t peers = match_digit(d, valid);
        if (valid && lane == __ffsll((unsigned long long)peers) - 1) atomicAdd(&L.base[d], (uint32_t)__popcll(peers));
    }
    __syncthreads();
    const uint32_t h = tid < kRadix ? L.base[tid] : 0u;
    if (tid < kRadix && h == (uint32_t)n) L.flag[pass] = 1u;
    const uint32_t b = block_exclusive_scan_fast(h, L.wsum);
    if (tid < kRadix) {
        L.base[tid] = b;
#pragma unroll
        for (int w = 0; w < NW; ++w) L.wc[w][tid] = 0;
    }
    __syncthreads();
    if (L.flag[pass]) return false;
    for (int c = 0; c < n; c += NT) {
        const int i = c + tid;
        const bool valid = i < n;
        const uint32_t key = valid ? sk[i] : 0u, val = valid ? sv[i] : 0u;
        const uint32_t d = (key >> shift) & (kRadix - 1);
        const uint64_t peers = match_digit(d, valid);
        const uint64_t below = peers & ((1ull << lane) - 1ull);
        if (valid && below == 0ull) L.wc[wave][d] = (uint32_t)__popcll(peers);
        __syncthreads();
        if (valid) {
            uint32_t pre = 0;
            for (int w = 0; w < wave; ++w) pre += L.wc[w][d];
            const uint32_t pos = L.base[d] + pre + (uint32_t)__popcll(below);
            dk[pos] = key;
            dv[pos] = val;
        }
        __syncthreads();
        if (tid < kRadix) {
            uint32_t placed = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                placed += L.wc[w][tid];
                L.wc[w][tid] = 0;
            }
            L.base[tid] += placed;
        }
        __syncthreads();
    }
    return true;
}

// Four passes; the result ends in (xk, xv) whichever passes were skipped.
template <int NW, bool kReg>
__device__ __forceinline__ void seg_sort(uint32_t* xk, uint32_t* xv, uint32_t* yk, uint32_t* yv, int n,
                                         SegShared<NW>& L) {
    bool in_x = true;
    for (int p = 0; p < 4; ++p) {
        bool moved;
        if (kReg)
            moved = in_x ? seg_pass_reg<NW>(xk, xv, yk, yv, n, p, L) : seg_pass_reg<NW>(yk, yv, xk, xv, n, p, L);
        else
            moved = in_x ? seg_pass_chunked<NW>(xk, xv, yk, yv, n, p, L)
                         : seg_pass_chunked<NW>(yk, yv, xk, xv, n, p, L);
        if (moved) in_x = !in_x;
    }
    if (!in_x) {
        for (int i = threadIdx.x; i < n; i += NW * 64) {
            xk[i] = yk[i];
            xv[i] = yv[i];
        }
        __syncthreads();
    }
}

template <int NW, int kLo, int kCap, bool kGlobalBeyond>
__device__ __forceinline__ void segment_sort_block(const uint32_t* __restrict__ seg_ranges,
                                                   const uint64_t* __restrict__ keys_in,
                                                   const uint32_t* __restrict__ vals_in,
                                                   uint64_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out,
                                                   uint32_t* gk0, uint32_t* gv0, uint32_t* gk1, uint32_t* gv1,
                                                   SegShared<NW>& L, uint32_t (*s_k)[kCap],
                                                   uint32_t (*s_v)[kCap]) {
    constexpr int NT = NW * 64;
    const int t = blockIdx.x;
    const uint32_t start = seg_ranges[2 * t], end = seg_ranges[2 * t + 1];
    const int n = (int)(end - start);
    if (n <= kLo || (!kGlobalBeyond && n > kCap)) return;
    const uint64_t hi = keys_in[start] & 0xFFFFFFFF00000000ull;
    if (threadIdx.x < 4) L.flag[threadIdx.x] = 0u;
    if (n <= kCap) {
        for (int i = threadIdx.x; i < n; i += NT) {
            s_k[0][i] = (uint32_t)keys_in[start + i];
            s_v[0][i] = vals_in[start + i];
        }
        __syncthreads();
        seg_sort<NW, true>(s_k[0], s_v[0], s_k[1], s_v[1], n, L);
        for (int i = threadIdx.x; i < n; i += NT) {
            keys_out[start + i] = hi | s_k[0][i];
            vals_out[start + i] = s_v[0][i];
        }
    } else {
        uint32_t* xk = gk0 + start; uint32_t* xv = gv0 + start;
        uint32_t* yk = gk1 + start; uint32_t* yv = gv1 + start;
        for (int i = threadIdx.x; i < n; i += NT) {
            xk[i] = (uint32_t)keys_in[start + i];
            xv[i] = vals_in[start + i];
        }
        __syncthreads();
        seg_sort<NW, false>(xk, xv, yk, yv, n, L);
        for (int i = threadIdx.x; i < n; i += NT) {
            keys_out[start + i] = hi | xk[i];
            vals_out[start + i] = xv[i];
        }
    }
}

constexpr int kSegMidCap = 4 * 64 * kSegRounds;    // 2048
constexpr int kSegBigCap = 16 * 64 * kSegRounds;   // 8192

__global__ __launch_bounds__(256) void k_segment_sort_mid(
    const uint32_t* __restrict__ seg_ranges, const uint64_t* __restrict__ keys_in,
    const uint32_t* __restrict__ vals_in, uint64_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out) {
    __shared__ SegShared<4> L;
    __shared__ uint32_t s_k[2][kSegMidCap];
    __shared__ uint32_t s_v[2][kSegMidCap];
    segment_sort_block<4, kSegWaveCap, kSegMidCap, false>(seg_ranges, keys_in, vals_in, keys_out, vals_out,
                                                          nullptr, nullptr, nullptr, nullptr, L, s_k, s_v);
}

__global__ __launch_bounds__(1024) void k_segment_sort_big(
    const uint32_t* __restrict__ seg_ranges, const uint64_t* __restrict__ keys_in,
    const uint32_t* __restrict__ vals_in, uint64_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out,
    uint32_t* __restrict__ gk0, uint32_t* __restrict__ gv0, uint32_t* __restrict__ gk1,
    uint32_t* __restrict__ gv1) {
    __shared__ SegShared<16> L;
    __shared__ uint32_t s_k[2][kSegBigCap];
    __shared__ uint32_t s_v[2][kSegBigCap];
    segment_sort_block<16, kSegMidCap, kSegBigCap, true>(seg_ranges, keys_in, vals_in, keys_out, vals_out,
                                                         gk0, gv0, gk1, gv1, L, s_k, s_v);
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

size_t bin_scratch_layout(int n, int64_t capacity, int n_tiles, BinScratch* out, void* base) {
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
    const size_t o_sr = take((size_t)n_tiles * 8);
    const size_t o_k0 = take((size_t)capacity * 4);
    const size_t o_v0 = take((size_t)capacity * 4);
    const size_t o_k1 = take((size_t)capacity * 4);
    const size_t o_v1 = take((size_t)capacity * 4);
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
        out->seg_ranges = (uint32_t*)(b + o_sr);
        out->seg_k0 = (uint32_t*)(b + o_k0);
        out->seg_v0 = (uint32_t*)(b + o_v0);
        out->seg_k1 = (uint32_t*)(b + o_k1);
        out->seg_v1 = (uint32_t*)(b + o_v1);
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

int tile_pass_count(int tile_bits) { return (tile_bits + 7) / 8; }

bool dup_writes_tmp(int tile_bits) { return (tile_pass_count(tile_bits) & 1) == 0; }

hipError_t launch_sort(uint64_t* keys, uint32_t* values, uint32_t n, int tile_bits, int n_tiles,
                       const BinScratch& s, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const int passes = tile_pass_count(tile_bits);
    // the tile-id passes end in the tmp pair; the per-tile sort writes (keys, values)
    uint64_t* kin = (passes & 1) ? keys : s.keys_tmp;
    uint32_t* vin = (passes & 1) ? values : s.vals_tmp;
    uint64_t* kout = (passes & 1) ? s.keys_tmp : keys;
    uint32_t* vout = (passes & 1) ? s.vals_tmp : values;
    const int nblk = (int)((n + kSortTile - 1) / kSortTile);
    for (int p = 0; p < passes; ++p) {
        const int shift = 32 + 8 * p;
        hipLaunchKernelGGL(k_digit_count, dim3(nblk), dim3(kSortThreads), 0, stream, kin, n, shift,
                           nblk, s.counts);
        hipLaunchKernelGGL(k_digit_scan, dim3(kRadix), dim3(256), 0, stream, s.counts, nblk,
                           s.digit_totals);
        hipLaunchKernelGGL(k_scatter, dim3(nblk), dim3(kSortThreads), 0, stream, kin, vin, n, shift,
                           nblk, s.counts, s.digit_totals, kout, vout);
        uint64_t* tk = kin; kin = kout; kout = tk;
        uint32_t* tv = vin; vin = vout; vout = tv;
    }
    // kin/vin now is the tmp pair, grouped by tile
    hipError_t e = launch_tile_ranges(s.keys_tmp, n, n_tiles, s.seg_ranges, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_segment_sort_wave, dim3((n_tiles + 3) / 4), dim3(256), 0, stream, s.seg_ranges,
                       n_tiles, s.keys_tmp, s.vals_tmp, keys, values);
    if (n > (uint32_t)kSegWaveCap)  // only then can a tile exceed the wave class
        hipLaunchKernelGGL(k_segment_sort_mid, dim3(n_tiles), dim3(256), 0, stream, s.seg_ranges,
                           s.keys_tmp, s.vals_tmp, keys, values);
    if (n > (uint32_t)kSegMidCap)
        hipLaunchKernelGGL(k_segment_sort_big, dim3(n_tiles), dim3(1024), 0, stream, s.seg_ranges,
                           s.keys_tmp, s.vals_tmp, keys, values, s.seg_k0, s.seg_v0, s.seg_k1, s.seg_v1);
    return hipGetLastError();
}

hipError_t launch_tile_ranges(const uint64_t* keys, uint32_t n_entries, int n_tiles,
                              uint32_t* ranges, hipStream_t stream) {
    // clear every tile (empty tiles keep (0, 0)), then mark the run boundaries
    const size_t words = 2 * (size_t)n_tiles;
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                       ranges, words, 0u);
    if (n_entries > 0)
        hipLaunchKernelGGL(k_ranges, dim3((n_entries + 255) / 256), dim3(256), 0, stream, keys,
                           n_entries, ranges);
    return hipGetLastError();
}

}  // namespace gs
