// Binning: a stable depth order of the splats, a prefix scan of their tile
// counts in that order, duplication into (tile_id << 32 | depth bits) keys,
// a stable sort on the tile bits, and tile ranges.
//
// Follows "rigel" README "Binning" (count, a scan giving every Gaussian a
// private slice, expansion, a sort restricted to the bits that can vary,
// a range kernel); zenn 4.1 (hierarchical exclusive scan), 4.2 (duplicate
// into the slice), 4.3 (8-bit LSD radix passes: histogram, bin starts,
// per-workgroup bin offsets, in-bin rank from the flag bits set before a
// lane, ping-pong buffers), 4.4 (range boundaries, empty tiles cleared);
// learn-gs build_tile_lists (span order, ty outer, tx inner) and prep_splats
// (which orders splats by depth before binning).
//
// Order. The required order is that of one stable sort of the entries by
// the 64-bit key, emitted Gaussian by Gaussian in index order: (tile, depth
// bits, Gaussian index). It is produced in two smaller sorts:
//   1. the N splats are sorted stably by depth bits (4 passes over N, not
//      over the entries; culled splats go last);
//   2. entries are emitted splat by splat in that order, so within any tile
//      they already appear in (depth bits, index) order;
//   3. one stable sort on the tile-id bits alone (two 8-bit passes at
//      1080p) then gives (tile, depth bits, index).
//
// MI355X design:
//  * Each radix pass is one kernel, a chained scan with decoupled look-back:
//    a workgroup takes a ticket from an atomic counter (so it only ever
//    waits for workgroups that started before it and are running), ranks
//    its 2048 keys, publishes its per-digit counts, looks back over
//    predecessors' published counts for its exclusive prefix and scatters.
//    Digit totals for every pass come from one histogram sweep. Every wait
//    is bounded: past the limit the workgroup records an error and stops
//    waiting, so no launch can hang.
//  * The in-workgroup rank uses 64-lane ballots: eight ballots, one per
//    digit bit, give each lane the mask of lanes holding its digit (there is
//    no match instruction on this architecture); popcount below the lane is
//    its rank (the zenn flag-bit rank). Per-wave LDS counters carry the rank
//    across rounds, so the order stays stable. Each workgroup stages its
//    output in LDS and writes per-digit runs, so global writes coalesce.
//  * The scan is reduce / scan-of-block-sums / rescan into per-splat
//    offsets. The duplication is entry-parallel: each workgroup takes 2048
//    consecutive entries, finds the splats that own them, stages their
//    offsets in LDS and gives every lane one entry, so the work is balanced
//    however many tiles a splat covers, and the stores coalesce.
#include <algorithm>

#include "gs_internal.h"

namespace gs {
namespace {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 8;
constexpr int kScanTile = kScanThreads * kScanItems;  // splats per workgroup

constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kEntryItems = 8;                          // entry keys per lane
constexpr int kEntryTile = kSortThreads * kEntryItems;  // entries per workgroup
constexpr int kGaussItems = 2;                          // splat keys per lane
constexpr int kGaussTile = kSortThreads * kGaussItems;  // splats per workgroup
constexpr int kRadix = 256;
constexpr int kGaussPasses = 4;                         // 32 depth bits
constexpr int kMaxTilePasses = 3;                       // up to 24 tile-id bits
constexpr int kTickets = 16;                            // tickets of every pass, error word last
constexpr int kLookBack = 8;                            // predecessors read per round trip

// look-back status words: (flag << 32) | count
constexpr uint64_t kFlagAggregate = 1ull << 32;
constexpr uint64_t kFlagPrefix = 2ull << 32;
constexpr int kSpinLimit = 1 << 20;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Inclusive scan of one value per thread across a 256-thread workgroup
// (Hillis-Steele in LDS). `tmp` holds 256 words. *total = the sum.
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

// Exclusive scan of one value per thread over a 256-thread workgroup: a
// shuffle scan in each wave, then one barrier for the wave totals. `wsum`
// holds 4 words and must not be in use by a previous call still being read.
__device__ __forceinline__ uint32_t block_exclusive_scan_fast(uint32_t x, uint32_t* wsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t v = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)v, off, 64);
        if (lane >= off) v += y;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    uint32_t pre = 0;
    for (int w = 0; w < wave; ++w) pre += wsum[w];
    return pre + v - x;
}

// Mask of the lanes of this wave that hold the same 8-bit digit (only valid
// lanes take part). All 64 lanes must be active.
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

template <typename K>
__device__ __forceinline__ uint32_t digit_of(K key, int shift) {
    return (uint32_t)(key >> shift) & (kRadix - 1);
}

// ---- scan (in a given order of the splats) ----

// counts are read as counts[perm[i]]: the i-th splat of the depth order.
__global__ __launch_bounds__(kScanThreads) void k_scan_reduce(const uint32_t* __restrict__ counts,
                                                              const uint32_t* __restrict__ perm, int n,
                                                              uint32_t* __restrict__ block_sums) {
    __shared__ uint32_t s_red[kScanThreads / 64];
    const int base = blockIdx.x * kScanTile;
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const int idx = base + i * kScanThreads + threadIdx.x;
        if (idx < n) sum += counts[perm[idx]];
    }
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
// The entry count goes to *total (and *n_dev if given); if an earlier
// radix pass gave up a wait (*err), the count is replaced by kCountFailed so
// that every later stage treats the frame as overflowed and writes nothing.
__global__ __launch_bounds__(1024) void k_scan_block_sums(const uint32_t* __restrict__ block_sums,
                                                          int nb, uint64_t* __restrict__ block_offsets,
                                                          uint64_t* __restrict__ total,
                                                          const uint32_t* __restrict__ err,
                                                          uint64_t* __restrict__ n_dev) {
    __shared__ uint64_t s[1024];
    constexpr int kPer = 8;
    const int tid = threadIdx.x;
    uint64_t local[kPer];
    uint64_t mine = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int idx = tid * kPer + i;
        local[i] = idx < nb ? (uint64_t)block_sums[idx] : 0;
        mine += local[i];
    }
    uint64_t sum = mine;
    s[tid] = sum;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        uint64_t y = tid >= off ? s[tid - off] : 0;
        __syncthreads();
        sum += y;
        s[tid] = sum;
        __syncthreads();
    }
    uint64_t run = sum - mine;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int idx = tid * kPer + i;
        if (idx < nb) block_offsets[idx] = run;
        run += local[i];
    }
    if (tid == 1023) {
        const uint64_t t = *err ? kCountFailed : sum;
        *total = t;
        if (n_dev) *n_dev = t;
    }
}

// offsets[i]: first entry of the i-th splat of the depth order.
__global__ __launch_bounds__(kScanThreads) void k_scan_offsets(const uint32_t* __restrict__ counts,
                                                               const uint32_t* __restrict__ perm, int n,
                                                               const uint64_t* __restrict__ block_offsets,
                                                               uint32_t* __restrict__ offsets) {
    __shared__ uint32_t s_c[kScanTile];
    __shared__ uint32_t s_tmp[kScanThreads];
    const int tid = threadIdx.x;
    const int base = blockIdx.x * kScanTile;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
        const int idx = i * kScanThreads + tid;
        s_c[idx] = base + idx < n ? counts[perm[base + idx]] : 0u;
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

// ---- duplication ----

// Entries a stage may touch: the count if it fits the caller's capacity,
// else none (the caller sees the count and grows its buffers).
__device__ __forceinline__ uint32_t usable_entries(const uint64_t* __restrict__ total, uint32_t capacity) {
    const uint64_t e = *total;
    return e <= (uint64_t)capacity ? (uint32_t)e : 0u;
}

// Last index i in [lo, hi] with offsets[i] <= e (offsets is nondecreasing;
// the answer owns entry e and never has a zero count).
__device__ __forceinline__ int owner_search(const uint32_t* __restrict__ offsets, int lo, int hi, uint32_t e) {
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offsets[mid] <= e) lo = mid; else hi = mid - 1;
    }
    return lo;
}

constexpr int kDupThreads = 256;
constexpr int kDupItems = 8;
constexpr int kDupTile = kDupThreads * kDupItems;
constexpr int kDupWindow = 2048;  // staged offsets; longer owner ranges search global memory
static_assert(kDupTile == kEntryTile, "a duplication workgroup fills exactly one sort tile");

// Per-workgroup digit counts, written as counts[(p * 256 + d) * nblk + b],
// and clearing of the look-back words of passes 1.. for this tile. `s_hist`
// is [passes][256], filled by the caller.
__device__ __forceinline__ void emit_counts(const uint32_t (*s_hist)[kRadix], int passes, int nblk,
                                            uint32_t* __restrict__ counts, uint64_t* __restrict__ status) {
    const int tid = threadIdx.x, b = blockIdx.x;
    for (int p = 0; p < passes; ++p) {
        counts[((size_t)p * kRadix + tid) * nblk + b] = s_hist[p][tid];
        if (p > 0) status[((size_t)(p - 1) * nblk + b) * kRadix + tid] = 0ull;
    }
}

// Entry e of the i-th splat g = perm[i] (its k-th tile, k = e - offsets[i])
// is the tile (x0 + k % w, y0 + k / w) of g's span. Each workgroup covers
// 2048 consecutive entries (one tile of the later sort); it finds the range
// of splats owning them, stages their offsets in LDS and searches there. It
// also counts the tile-id digits of its entries for every radix pass.
__global__ __launch_bounds__(kDupThreads) void k_duplicate(
    const float4* __restrict__ xy_depth, const uint32_t* __restrict__ offsets,
    const uint32_t* __restrict__ perm, int n, const uint64_t* __restrict__ total, uint32_t capacity, int TX,
    int TY, int passes, uint64_t* __restrict__ keys, uint32_t* __restrict__ values,
    uint32_t* __restrict__ counts, uint64_t* __restrict__ status) {
    __shared__ uint32_t s_off[kDupWindow];
    __shared__ uint32_t s_hist[kMaxTilePasses][kRadix];
    __shared__ int s_range[2];
    const int tid = threadIdx.x, lane = tid & 63;
    const uint32_t n_entries = usable_entries(total, capacity);
    const uint32_t e0 = blockIdx.x * kDupTile;
    if (e0 >= n_entries) return;  // the grid is sized for the capacity
    const uint32_t e1 = min(e0 + (uint32_t)kDupTile, n_entries);
#pragma unroll
    for (int p = 0; p < kMaxTilePasses; ++p) s_hist[p][tid] = 0;
    if (tid < 2) s_range[tid] = owner_search(offsets, 0, n - 1, tid == 0 ? e0 : e1 - 1);
    __syncthreads();
    const int i_lo = s_range[0], i_hi = s_range[1];
    const int span = i_hi - i_lo + 1;
    const bool staged = span <= kDupWindow;
    if (staged)
        for (int i = tid; i < span; i += kDupThreads) s_off[i] = offsets[i_lo + i];
    __syncthreads();
#pragma unroll 2
    for (int it = 0; it < kDupItems; ++it) {
        const uint32_t e = e0 + it * kDupThreads + tid;
        const bool valid = e < e1;
        uint32_t t = 0;
        if (valid) {
            int i;
            uint32_t off;
            if (staged) {
                int lo = 0, hi = span - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (s_off[mid] <= e) lo = mid; else hi = mid - 1;
                }
                i = i_lo + lo;
                off = s_off[lo];
            } else {
                i = owner_search(offsets, i_lo, i_hi, e);
                off = offsets[i];
            }
            const uint32_t g = perm[i];
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
            t = ty * (uint32_t)TX + tx;
            keys[e] = ((uint64_t)t << 32) | (uint64_t)__float_as_uint(rec.z);
            values[e] = g;
        }
        for (int p = 0; p < passes; ++p) {
            const uint32_t d = (t >> (8 * p)) & (kRadix - 1);
            const uint64_t peers = match_digit(d, valid);
            if (valid && lane == __ffsll((unsigned long long)peers) - 1)
                atomicAdd(&s_hist[p][d], (uint32_t)__popcll(peers));
        }
    }
    __syncthreads();
    emit_counts(s_hist, passes, (int)gridDim.x, counts, status);
}

// ---- radix sort ----

// Depth keys of the splats (culled ones last), the identity permutation and
// the per-tile digit counts of all four depth passes. Workgroup 0 also
// clears the tickets and the error word of every pass of this call.
__global__ __launch_bounds__(kSortThreads) void k_depth_keys(const float4* __restrict__ xy_depth,
                                                             const uint32_t* __restrict__ tiles_touched,
                                                             int n, uint32_t* __restrict__ keys,
                                                             uint32_t* __restrict__ vals,
                                                             uint32_t* __restrict__ counts,
                                                             uint64_t* __restrict__ status,
                                                             uint32_t* __restrict__ tickets) {
    __shared__ uint32_t s_hist[kGaussPasses][kRadix];
    const int tid = threadIdx.x, lane = tid & 63;
    if (blockIdx.x == 0 && tid < kTickets) tickets[tid] = 0u;
#pragma unroll
    for (int p = 0; p < kGaussPasses; ++p) s_hist[p][tid] = 0;
    __syncthreads();
    const int base = blockIdx.x * kGaussTile;
#pragma unroll
    for (int i = 0; i < kGaussItems; ++i) {
        const int g = base + i * kSortThreads + tid;
        const bool valid = g < n;
        uint32_t key = 0xFFFFFFFFu;
        if (valid) {
            if (tiles_touched[g] != 0u) key = __float_as_uint(xy_depth[g].z);
            keys[g] = key;
            vals[g] = (uint32_t)g;
        }
#pragma unroll
        for (int p = 0; p < kGaussPasses; ++p) {
            const uint32_t d = digit_of(key, 8 * p);
            const uint64_t peers = match_digit(d, valid);
            if (valid && lane == __ffsll((unsigned long long)peers) - 1)
                atomicAdd(&s_hist[p][d], (uint32_t)__popcll(peers));
        }
    }
    __syncthreads();
    emit_counts(s_hist, kGaussPasses, (int)gridDim.x, counts, status);
}

// Rows r = p * 256 + d of counts (one per pass and digit, row stride
// `stride`): hist[r] = the total of the row's first nblk tiles; rows of pass
// 0 are replaced in place by their exclusive prefix over tiles. nblk covers
// the usable entries (*total, capacity) when total is given. One wave per row.
__global__ __launch_bounds__(256) void k_count_scan(uint32_t* __restrict__ counts, int stride, int nblk,
                                                    const uint64_t* __restrict__ total, uint32_t capacity,
                                                    int tile_keys, int rows, uint32_t* __restrict__ hist) {
    const int lane = threadIdx.x & 63;
    const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;  // whole waves
    if (total) nblk = (int)((usable_entries(total, capacity) + (uint32_t)tile_keys - 1) / (uint32_t)tile_keys);
    uint32_t* row = counts + (size_t)r * stride;
    const int per = (nblk + 63) / 64;
    const int i0 = min(lane * per, nblk), i1 = min(i0 + per, nblk);
    uint32_t sum = 0;
    for (int i = i0; i < i1; ++i) sum += row[i];
    uint32_t incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)incl, off, 64);
        if (lane >= off) incl += y;
    }
    if (r < kRadix) {
        uint32_t run = incl - sum;
        for (int i = i0; i < i1; ++i) {
            const uint32_t c = row[i];
            row[i] = run;
            run += c;
        }
    }
    const uint32_t row_total = (uint32_t)__shfl((int)incl, 63, 64);
    if (lane == 0) hist[r] = row_total;
}

// One stable radix pass over n (key, value) pairs on digit (key >> shift),
// 256 * ITEMS keys per workgroup.
//   hist     [256] digit totals of this pass
//   prefix   if not NULL: [256][nblk] exclusive per-tile prefixes of each
//            digit (known in advance for the first pass); else the prefixes
//            come from a look-back over:
//   status   [nblk][256] look-back words, zero on entry
//   ticket   workgroup order counter, zero on entry
//   err      set to 1 if a wait ever exceeded its bound; *fail_dev (if
//            given) is then set to kCountFailed as well
// The key count is n, or the usable entries (*total, capacity) when total
// is given (the grid is then sized for the capacity; idle workgroups exit).
template <typename K, int ITEMS>
__global__ __launch_bounds__(kSortThreads) void k_onesweep(
    const K* __restrict__ keys_in, const uint32_t* __restrict__ vals_in, uint32_t n,
    const uint64_t* __restrict__ total, uint32_t capacity, int shift, const uint32_t* __restrict__ hist,
    const uint32_t* __restrict__ prefix, uint64_t* __restrict__ status, uint32_t* __restrict__ ticket,
    uint32_t* __restrict__ err, uint64_t* __restrict__ fail_dev, K* __restrict__ keys_out,
    uint32_t* __restrict__ vals_out) {
    constexpr int kTileKeys = kSortThreads * ITEMS;
    __shared__ uint32_t s_wcount[kSortWaves][kRadix];  // per-wave digit counts, then prefixes
    __shared__ uint32_t s_local_start[kRadix];
    __shared__ uint32_t s_gbase[kRadix];
    __shared__ uint32_t s_wsum[2][4];
    __shared__ uint32_t s_block;
    __shared__ K s_keys[kTileKeys];
    __shared__ uint32_t s_vals[kTileKeys];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) s_block = prefix ? blockIdx.x : atomicAdd(ticket, 1u);
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) s_wcount[w][tid] = 0;
    __syncthreads();
    const uint32_t b = s_block;
    const uint32_t base = b * kTileKeys;
    if (total) n = usable_entries(total, capacity);
    if (base >= n) return;  // whole workgroup

    // stable rank of every key among equal digits of this workgroup's tile
    K key[ITEMS];
    uint32_t val[ITEMS];
    uint32_t rank[ITEMS];
    const uint32_t seg = base + wave * (64 * ITEMS);
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const uint32_t pos = seg + i * 64 + lane;
        const bool valid = pos < n;
        key[i] = valid ? keys_in[pos] : K(0);
        val[i] = valid ? vals_in[pos] : 0u;
    }
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const bool valid = seg + i * 64 + lane < n;
        const uint32_t d = digit_of(key[i], shift);
        const uint64_t peers = match_digit(d, valid);
        const uint64_t below = peers & ((1ull << lane) - 1ull);
        uint32_t before = 0;
        if (valid) before = s_wcount[wave][d];
        rank[i] = before + (uint32_t)__popcll(below);
        if (valid && below == 0ull) s_wcount[wave][d] = before + (uint32_t)__popcll(peers);
    }
    __syncthreads();

    // digit d = tid: wave prefixes, the tile's own count, its local start
    const int d = tid;
    uint32_t count = 0;
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) {
        const uint32_t c = s_wcount[w][d];
        s_wcount[w][d] = count;
        count += c;
    }
    s_local_start[d] = block_exclusive_scan_fast(count, s_wsum[0]);
    const uint32_t dstart = block_exclusive_scan_fast(hist[d], s_wsum[1]);

    uint32_t excl = 0;
    if (prefix) {
        excl = prefix[(size_t)d * gridDim.x + b];
    } else {
        // publish this tile's count, look back for the exclusive prefix,
        // eight predecessors' words per round trip
        uint64_t* mine = status + (size_t)b * kRadix + d;
        if (b == 0) {
            __hip_atomic_store(mine, kFlagPrefix | count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            __hip_atomic_store(mine, kFlagAggregate | count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            int j = (int)b - 1;
            int spins = 0;
            bool done = false;
            while (!done) {
                uint64_t w8[kLookBack];
#pragma unroll
                for (int k = 0; k < kLookBack; ++k)
                    w8[k] = j - k >= 0 ? __hip_atomic_load(status + (size_t)(j - k) * kRadix + d, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT)
                                       : kFlagPrefix;
#pragma unroll
                for (int k = 0; k < kLookBack; ++k) {
                    if (done) break;
                    uint64_t v = w8[k];
                    while ((v >> 32) == 0ull) {
                        if (++spins > kSpinLimit) {  // never expected: give up rather than hang
                            __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            if (fail_dev)
                                __hip_atomic_store(fail_dev, kCountFailed, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
                            v = kFlagPrefix;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(1);
                        v = __hip_atomic_load(status + (size_t)(j - k) * kRadix + d, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
                    }
                    excl += (uint32_t)v;
                    done = (v >> 32) == 2ull;
                }
                j -= kLookBack;
            }
            __hip_atomic_store(mine, kFlagPrefix | (excl + count), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    s_gbase[d] = dstart + excl;
    __syncthreads();

    // stage in digit order, write out per-digit runs
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const uint32_t pos = seg + i * 64 + lane;
        if (pos < n) {
            const uint32_t dd = digit_of(key[i], shift);
            const uint32_t slot = s_local_start[dd] + s_wcount[wave][dd] + rank[i];
            s_keys[slot] = key[i];
            s_vals[slot] = val[i];
        }
    }
    __syncthreads();
    const uint32_t valid_n = min(n - base, (uint32_t)kTileKeys);
    for (uint32_t s = tid; s < valid_n; s += kSortThreads) {
        const K k = s_keys[s];
        const uint32_t dd = digit_of(k, shift);
        const uint32_t out = s_gbase[dd] + (s - s_local_start[dd]);
        keys_out[out] = k;
        vals_out[out] = s_vals[s];
    }
}

// ---- tile ranges ----

__global__ void k_fill_u32(uint32_t* __restrict__ p, size_t n, uint32_t v) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// Run boundaries of the sorted tile ids. The count is n, or the usable
// entries (*total, capacity) when total is given.
__global__ void k_ranges(const uint64_t* __restrict__ keys, uint32_t n, const uint64_t* __restrict__ total,
                         uint32_t capacity, uint32_t* __restrict__ ranges) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (total) n = usable_entries(total, capacity);
    if (i >= n) return;
    const uint32_t t = (uint32_t)(keys[i] >> 32);
    if (i == 0 || (uint32_t)(keys[i - 1] >> 32) != t) ranges[2 * (size_t)t] = i;
    if (i == n - 1 || (uint32_t)(keys[i + 1] >> 32) != t) ranges[2 * (size_t)t + 1] = i + 1;
}

int tile_pass_count(int tile_bits) { return (tile_bits + 7) / 8; }

}  // namespace

size_t bin_scratch_layout(int n, int64_t capacity, BinScratch* out, void* base) {
    const size_t nb_scan = (size_t)(n + kScanTile - 1) / kScanTile;
    const size_t nb_gauss = (size_t)(n + kGaussTile - 1) / kGaussTile;
    const size_t nb_entry = (size_t)((capacity + kEntryTile - 1) / kEntryTile);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align256(bytes > 0 ? bytes : 1);
        return at;
    };
    // tickets of every pass and the error word (word 15), cleared by the
    // first kernel of every call, then the entry count, so the host reads
    // the error word and the count with one copy
    const size_t o_tick = take(kTickets * 4 + 8);
    const size_t o_ghist = take((size_t)kGaussPasses * kRadix * 4);
    const size_t o_ehist = take((size_t)kMaxTilePasses * kRadix * 4);
    const size_t o_gcnt = take(nb_gauss * kRadix * kGaussPasses * 4);
    const size_t o_ecnt = take(nb_entry * kRadix * kMaxTilePasses * 4);
    // look-back words of passes 1.., cleared by the kernels that count
    const size_t o_gstat = take(nb_gauss * kRadix * (kGaussPasses - 1) * 8);
    const size_t o_estat = take(nb_entry * kRadix * (kMaxTilePasses - 1) * 8);
    const size_t o_bs = take(nb_scan * 4);
    const size_t o_bo = take(nb_scan * 8);
    const size_t o_off = take((size_t)n * 4);
    const size_t o_gk0 = take((size_t)n * 4);
    const size_t o_gv0 = take((size_t)n * 4);
    const size_t o_gk1 = take((size_t)n * 4);
    const size_t o_gv1 = take((size_t)n * 4);
    const size_t o_kt = take((size_t)capacity * 8);
    const size_t o_vt = take((size_t)capacity * 4);
    if (out && base) {
        char* b = (char*)base;
        out->tickets = (uint32_t*)(b + o_tick);
        out->err = out->tickets + (kTickets - 1);
        out->total = (uint64_t*)(b + o_tick + kTickets * 4);
        out->gauss_hist = (uint32_t*)(b + o_ghist);
        out->entry_hist = (uint32_t*)(b + o_ehist);
        out->gauss_counts = (uint32_t*)(b + o_gcnt);
        out->entry_counts = (uint32_t*)(b + o_ecnt);
        out->gauss_status = (uint64_t*)(b + o_gstat);
        out->entry_status = (uint64_t*)(b + o_estat);
        out->block_sums = (uint32_t*)(b + o_bs);
        out->block_offsets = (uint64_t*)(b + o_bo);
        out->offsets = (uint32_t*)(b + o_off);
        out->gk[0] = (uint32_t*)(b + o_gk0);
        out->gv[0] = (uint32_t*)(b + o_gv0);
        out->gk[1] = (uint32_t*)(b + o_gk1);
        out->gv[1] = (uint32_t*)(b + o_gv1);
        out->keys_tmp = (uint64_t*)(b + o_kt);
        out->vals_tmp = (uint32_t*)(b + o_vt);
    }
    return off;
}

hipError_t launch_bin_and_sort(const gs_camera& cam, int n, const float4* xy_depth,
                               const uint32_t* tiles_touched, uint64_t* keys, uint32_t* values,
                               uint32_t capacity, const BinScratch& s, uint64_t* n_dev, hipStream_t stream) {
    // 1. stable depth order of the splats (culled last) into gv[0]
    const unsigned nbg = (unsigned)((n + kGaussTile - 1) / kGaussTile);
    hipLaunchKernelGGL(k_depth_keys, dim3(nbg), dim3(kSortThreads), 0, stream, xy_depth, tiles_touched, n,
                       s.gk[0], s.gv[0], s.gauss_counts, s.gauss_status, s.tickets);
    const int grows = kGaussPasses * kRadix;
    hipLaunchKernelGGL(k_count_scan, dim3((grows + 3) / 4), dim3(256), 0, stream, s.gauss_counts, (int)nbg,
                       (int)nbg, (const uint64_t*)nullptr, 0u, kGaussTile, grows, s.gauss_hist);
    for (int p = 0; p < kGaussPasses; ++p) {
        const int src = p & 1, dst = src ^ 1;  // an even pass count leaves the order in gv[0]
        hipLaunchKernelGGL((k_onesweep<uint32_t, kGaussItems>), dim3(nbg), dim3(kSortThreads), 0, stream,
                           s.gk[src], s.gv[src], (uint32_t)n, (const uint64_t*)nullptr, 0u, 8 * p,
                           s.gauss_hist + p * kRadix, p == 0 ? s.gauss_counts : nullptr,
                           p == 0 ? nullptr : s.gauss_status + (size_t)(p - 1) * nbg * kRadix, s.tickets + p,
                           s.err, n_dev, s.gk[dst], s.gv[dst]);
    }
    // 2. exclusive scan of the tile counts in depth order; E -> s.total
    const int nbs = (n + kScanTile - 1) / kScanTile;
    const uint32_t* perm = s.gv[0];
    hipLaunchKernelGGL(k_scan_reduce, dim3(nbs), dim3(kScanThreads), 0, stream, tiles_touched, perm, n,
                       s.block_sums);
    hipLaunchKernelGGL(k_scan_block_sums, dim3(1), dim3(1024), 0, stream, s.block_sums, nbs, s.block_offsets,
                       s.total, (const uint32_t*)s.err, n_dev);
    hipLaunchKernelGGL(k_scan_offsets, dim3(nbs), dim3(kScanThreads), 0, stream, tiles_touched, perm, n,
                       s.block_offsets, s.offsets);
    // 3. duplication and the stable sort on the tile-id bits. Grids cover the
    // capacity; the kernels read E and do nothing when it exceeds capacity.
    const unsigned nbe = (capacity + kEntryTile - 1) / kEntryTile;
    if (nbe == 0) return hipGetLastError();
    int tile_bits = 0;
    while ((1 << tile_bits) < tiles_x(cam) * tiles_y(cam)) ++tile_bits;
    const int passes = tile_pass_count(tile_bits);
    // entries start in the tmp pair when the pass count is odd, so the last
    // pass always writes (keys, values)
    uint64_t* kin = (passes & 1) ? s.keys_tmp : keys;
    uint32_t* vin = (passes & 1) ? s.vals_tmp : values;
    uint64_t* kout = (passes & 1) ? keys : s.keys_tmp;
    uint32_t* vout = (passes & 1) ? values : s.vals_tmp;
    hipLaunchKernelGGL(k_duplicate, dim3(nbe), dim3(kDupThreads), 0, stream, xy_depth, s.offsets, s.gv[0], n,
                       (const uint64_t*)s.total, capacity, tiles_x(cam), tiles_y(cam), passes, kin, vin,
                       s.entry_counts, s.entry_status);
    if (passes == 0) return hipGetLastError();
    const int erows = passes * kRadix;
    hipLaunchKernelGGL(k_count_scan, dim3((erows + 3) / 4), dim3(256), 0, stream, s.entry_counts, (int)nbe, 0,
                       (const uint64_t*)s.total, capacity, kEntryTile, erows, s.entry_hist);
    for (int p = 0; p < passes; ++p) {
        hipLaunchKernelGGL((k_onesweep<uint64_t, kEntryItems>), dim3(nbe), dim3(kSortThreads), 0, stream, kin,
                           vin, 0u, (const uint64_t*)s.total, capacity, 32 + 8 * p, s.entry_hist + p * kRadix,
                           p == 0 ? s.entry_counts : nullptr,
                           p == 0 ? nullptr : s.entry_status + (size_t)(p - 1) * nbe * kRadix,
                           s.tickets + kGaussPasses + p, s.err, n_dev, kout, vout);
        uint64_t* tk = kin; kin = kout; kout = tk;
        uint32_t* tv = vin; vin = vout; vout = tv;
    }
    return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, size_t words, uint32_t v, hipStream_t stream) {
    if (words == 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream, p, words, v);
    return hipGetLastError();
}

hipError_t launch_tile_ranges(const uint64_t* keys, uint32_t n_entries, const uint64_t* n_dev, uint32_t capacity,
                              int n_tiles, uint32_t* ranges, hipStream_t stream) {
    // clear every tile (empty tiles keep (0, 0)), then mark the run boundaries
    const size_t words = 2 * (size_t)n_tiles;
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                       ranges, words, 0u);
    const uint32_t grid_n = n_dev ? capacity : n_entries;
    if (grid_n > 0)
        hipLaunchKernelGGL(k_ranges, dim3((grid_n + 255) / 256), dim3(256), 0, stream, keys, n_entries, n_dev,
                           capacity, ranges);
    return hipGetLastError();
}

}  // namespace gs
