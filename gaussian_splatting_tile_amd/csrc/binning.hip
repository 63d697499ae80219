// Binning: a stable depth order of the splats, a prefix scan of their tile
// counts in that order, duplication into (tile_id << 32 | depth bits) keys,
// a stable sort on the tile bits, and tile ranges.
//
// Follows "rigel" README "Binning" (count, a scan giving every Gaussian a
// private slice, expansion, a sort restricted to the bits that can vary,
// a range kernel); zenn 4.1 (exclusive scan of the tile counts), 4.2 (duplicate
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
//   3. one stable sort on the tile-id bits alone (passes of at most 8 bits,
//      the bits split evenly: 7 + 6 for the 13 bits of a 1080p grid) then
//      gives (tile, depth bits, index).
//
// MI355X design:
//  * Each radix pass is reduce-then-scan with no waits between workgroups:
//    per-tile digit counts (LDS histograms, one column per tile), a small
//    kernel that turns them into per-tile exclusive prefixes and digit
//    totals (one wave per digit), and the pass itself, which ranks and
//    scatters its tile independently. The first pass's counts come from the
//    kernel that produces the keys; later passes count their input in a
//    kernel of their own. Two alternatives were measured and dropped: a
//    chained scan with decoupled look-back (its coherent polling across the
//    eight L2s cost more than the passes) and counting the next pass's
//    digits with global atomics while scattering (digits with few distinct
//    values serialise on a handful of counters).
//  * The in-workgroup rank uses 64-lane ballots: eight ballots, one per
//    digit bit, give each lane the mask of lanes holding its digit (there is
//    no match instruction on this architecture); popcount below the lane is
//    its rank (the zenn flag-bit rank). Per-wave LDS counters carry the rank
//    across rounds, so the order stays stable. Each workgroup stages its
//    output in LDS and writes per-digit runs, so global writes coalesce.
//  * The exclusive scan of tiles_touched in depth order rides on the last
//    depth pass: its counting kernel also sums tiles_touched per (tile,
//    digit), the prefix kernel scans those sums too, and the pass writes
//    each splat's first entry where it writes the splat itself, plus the
//    owner of every 2048-entry duplication tile's first entry and E.
//  * The duplication is entry-parallel: each workgroup takes 2048
//    consecutive entries (one tile of the later sort), derives the owner of
//    each entry from the owners' start slots with a max-scan in LDS and
//    gives every lane one entry, so the work is balanced however many tiles
//    a splat covers, and the stores coalesce.
#include <algorithm>

#include "gs_internal.h"

namespace gs {
namespace {

constexpr int kDupThreads = 256;
constexpr int kDupItems = 8;
constexpr int kDupTile = kDupThreads * kDupItems;  // entries per duplication workgroup

constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / 64;
constexpr int kEntryItems = 8;                          // entry keys per lane
constexpr int kEntryTile = kSortThreads * kEntryItems;  // entries per workgroup
// Splat keys per lane in the depth passes: 2 for small frames (enough
// workgroups to spread the latency-bound passes), 8 from kGaussBigN splats
// on (fewer, fuller workgroups: the per-workgroup scans and staging are
// amortised over four times the keys).
constexpr int kGaussItems = 2;
constexpr int kGaussItemsBig = 8;
#ifndef GS_DEPTH_BIG_N
#define GS_DEPTH_BIG_N (1 << 19)
#endif
constexpr int kGaussBigN = GS_DEPTH_BIG_N;
constexpr int kGaussTile = kSortThreads * kGaussItems;  // splats per workgroup (the smaller tile: scratch bound)
constexpr int kRadix = 256;
constexpr int kGaussPasses = 4;                         // 32 depth bits
constexpr int kMaxTilePasses = 3;                       // up to 24 tile-id bits

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

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

__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int off) {
    const uint32_t lo = (uint32_t)__shfl_up((int)(uint32_t)v, off, 64);
    const uint32_t hi = (uint32_t)__shfl_up((int)(uint32_t)(v >> 32), off, 64);
    return ((uint64_t)hi << 32) | lo;
}

// 64-bit version of block_exclusive_scan_fast; `wsum` holds 4 words.
__device__ __forceinline__ uint64_t block_exclusive_scan_u64(uint64_t x, uint64_t* wsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t v = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint64_t y = shfl_up_u64(v, off);
        if (lane >= off) v += y;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    uint64_t pre = 0;
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

// A pass's digit: `pass` packs the digit's shift (low 8 bits) and its
// width in bits (bits 8..11; 0 means the full 8).
template <typename K>
__device__ __forceinline__ uint32_t digit_of(K key, int pass) {
    const int width = (pass >> 8) != 0 ? (pass >> 8) : 8;
    return (uint32_t)(key >> (pass & 0xFF)) & ((1u << width) - 1u);
}
__host__ __device__ constexpr int digit_pass(int shift, int width) { return shift | (width << 8); }

// ---- duplication ----

// Entries a stage may touch: the count if it fits the caller's capacity,
// else none (the caller sees the count and grows its buffers).
__device__ __forceinline__ uint32_t usable_entries(const uint64_t* __restrict__ total, uint32_t capacity) {
    const uint64_t e = *total;
    return e <= (uint64_t)capacity ? (uint32_t)e : 0u;
}

static_assert(kDupTile == kEntryTile, "a duplication workgroup fills exactly one sort tile");

// This workgroup's column b of one pass's per-tile digit counts,
// counts[d * nblk + b], from the LDS histogram `s_hist`.
__device__ __forceinline__ void emit_counts(const uint32_t* s_hist, int nblk, uint32_t* __restrict__ counts) {
    counts[(size_t)threadIdx.x * nblk + blockIdx.x] = s_hist[threadIdx.x];
}

// Entry e of the i-th splat g = perm[i] (its k-th tile, k = e - offsets[i])
// is the tile (x0 + k % w, y0 + k / w) of g's span. Each workgroup covers
// 2048 consecutive entries (one tile of the later sort). Owners without a
// search: first_owner gives the owner i_lo of the first entry; every later
// splat whose entries start inside the tile marks its first slot (LDS max,
// so of several splats starting at one slot, the last, which is the one
// with entries, wins), and an inclusive max-scan over the 2048 slots gives
// every entry its owner. The workgroup also counts the first tile pass's
// digits of its entries.
template <bool ELLIPSE>
__global__ __launch_bounds__(kDupThreads) void k_duplicate(
    const float4* __restrict__ xy_depth, const float4* __restrict__ conic_op, const uint32_t* __restrict__ offsets,
    const uint32_t* __restrict__ perm, const uint32_t* __restrict__ first_owner, int n,
    const uint64_t* __restrict__ total, uint32_t capacity, int TX, int TY, uint32_t n_view, int passes,
    int first_pass, uint64_t* __restrict__ keys, uint32_t* __restrict__ values, uint32_t* __restrict__ counts) {
    constexpr int kPer = kDupTile / kDupThreads;  // slots per thread in the scan
    __shared__ uint32_t s_owner[kDupTile];
    __shared__ uint32_t s_hist[kRadix];
    __shared__ uint32_t s_wmax[kDupThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t n_entries = usable_entries(total, capacity);
    const uint32_t e0 = blockIdx.x * kDupTile;
    if (e0 >= n_entries) return;  // the grid is sized for the capacity
    const uint32_t e1 = min(e0 + (uint32_t)kDupTile, n_entries);
    const int i_lo = (int)first_owner[blockIdx.x];
    s_hist[tid] = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) s_owner[j * kDupThreads + tid] = 0u;
    __syncthreads();
    // splats after i_lo start strictly inside the tile until the first one at or past e1
    for (int i = i_lo + 1 + tid; i < n; i += kDupThreads) {
        const uint32_t off = offsets[i];
        if (off >= e1) break;
        atomicMax(&s_owner[off - e0], (uint32_t)(i - i_lo));
    }
    __syncthreads();
    // inclusive max-scan of s_owner: thread t holds slots [kPer t, kPer t + kPer)
    uint32_t v[kPer];
    uint32_t run = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        run = max(run, s_owner[tid * kPer + j]);
        v[j] = run;
    }
    uint32_t incl = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)incl, off, 64);
        if (lane >= off) incl = max(incl, y);
    }
    if (lane == 63) s_wmax[wave] = incl;
    uint32_t excl = (uint32_t)__shfl_up((int)incl, 1, 64);
    if (lane == 0) excl = 0;
    __syncthreads();
    for (int w = 0; w < wave; ++w) excl = max(excl, s_wmax[w]);
#pragma unroll
    for (int j = 0; j < kPer; ++j) s_owner[tid * kPer + j] = max(v[j], excl);
    __syncthreads();
#pragma unroll 2
    for (int it = 0; it < kDupItems; ++it) {
        const uint32_t slot = it * kDupThreads + tid;
        const uint32_t e = e0 + slot;
        const bool valid = e < e1;
        uint32_t t = 0;
        if (valid) {
            const int i = i_lo + (int)s_owner[slot];
            const uint32_t g = perm[i];
            const uint32_t k = e - offsets[i];
            const float4 rec = xy_depth[g];
            const Span sp = tile_span(rec.x, rec.y, rec.w, TX, TY);
            uint32_t tx, ty;
            if (ELLIPSE) {
                // the k-th kept tile, rows of kept runs in span order
                const float4 co = conic_op[g];
                const EllipseRows er = ellipse_rows(rec.x, rec.y, co.x, co.y, co.z, sp);
                int kk = (int)k, row = sp.y0, lo = sp.x0, hi = sp.x0;
                for (; row < sp.y1; ++row) {
                    ellipse_row_range(er, sp, row, lo, hi);
                    const int cnt = hi > lo ? hi - lo : 0;
                    if (kk < cnt) break;
                    kk -= cnt;
                }
                // row < sp.y1 always: k < tiles_touched, the count of the same runs;
                // the clamps keep any tile id inside the grid regardless
                tx = (uint32_t)max(sp.x0, min(lo + kk, sp.x1 - 1));
                ty = (uint32_t)min(row, sp.y1 - 1);
            } else {
                const uint32_t w = (uint32_t)(sp.x1 - sp.x0);
                // k / w and k % w: float quotient (k < 2^21) fixed up by one step
                uint32_t q = (uint32_t)((float)k * __builtin_amdgcn_rcpf((float)w));
                int r = (int)k - (int)(q * w);
                if (r < 0) { --q; r += (int)w; }
                if (r >= (int)w) { ++q; r -= (int)w; }
                tx = (uint32_t)sp.x0 + (uint32_t)r;
                ty = (uint32_t)sp.y0 + q;
            }
            // splat g of view g / n_view lists its tiles in that view's band
            const uint32_t band = g / n_view;
            t = (band * (uint32_t)TY + ty) * (uint32_t)TX + tx;
            keys[e] = ((uint64_t)t << 32) | (uint64_t)__float_as_uint(rec.z);
            values[e] = g;
        }
        if (passes > 0) {  // the first tile pass's digit: the low bits of the tile id
            const uint32_t d = digit_of((uint64_t)t << 32, first_pass);
            const uint64_t peers = match_digit(d, valid);
            if (valid && lane == __ffsll((unsigned long long)peers) - 1)
                atomicAdd(&s_hist[d], (uint32_t)__popcll(peers));
        }
    }
    __syncthreads();
    if (passes > 0) emit_counts(s_hist, (int)gridDim.x, counts);
}

// ---- radix sort ----

// Depth keys of the splats (culled ones last), the identity permutation and
// the per-tile counts of the first depth pass's digit.
template <int ITEMS>
__global__ __launch_bounds__(kSortThreads) void k_depth_keys(const float4* __restrict__ xy_depth,
                                                             const uint32_t* __restrict__ tiles_touched,
                                                             int n, uint32_t* __restrict__ keys,
                                                             uint32_t* __restrict__ vals,
                                                             uint32_t* __restrict__ counts) {
    __shared__ uint32_t s_hist[kRadix];
    const int tid = threadIdx.x, lane = tid & 63;
    s_hist[tid] = 0;
    __syncthreads();
    const int base = blockIdx.x * (kSortThreads * ITEMS);
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const int g = base + i * kSortThreads + tid;
        const bool valid = g < n;
        uint32_t key = 0xFFFFFFFFu;
        if (valid) {
            if (tiles_touched[g] != 0u) key = __float_as_uint(xy_depth[g].z);
            keys[g] = key;
            vals[g] = (uint32_t)g;
        }
        const uint32_t d = digit_of(key, 0);
        const uint64_t peers = match_digit(d, valid);
        if (valid && lane == __ffsll((unsigned long long)peers) - 1)
            atomicAdd(&s_hist[d], (uint32_t)__popcll(peers));
    }
    __syncthreads();
    emit_counts(s_hist, (int)gridDim.x, counts);
}

// Per-tile counts of digit (key >> shift) of the keys about to be sorted by
// a later pass: one tile of 256 * ITEMS keys per workgroup, as in the pass.
// The key count is n, or the usable entries (*total, capacity). With TT (the
// last depth pass) it also sums, per tile and digit, tiles_touched of the
// splats the keys belong to (vals), into tt_counts.
template <typename K, int ITEMS, bool TT>
__global__ __launch_bounds__(kSortThreads) void k_count_digits(const K* __restrict__ keys, uint32_t n,
                                                               const uint64_t* __restrict__ total,
                                                               uint32_t capacity, int shift,
                                                               uint32_t* __restrict__ counts,
                                                               const uint32_t* __restrict__ vals,
                                                               const uint32_t* __restrict__ tiles_touched,
                                                               uint32_t* __restrict__ tt_counts) {
    constexpr int kTileKeys = kSortThreads * ITEMS;
    __shared__ uint32_t s_hist[kRadix];
    __shared__ uint32_t s_tt[TT ? kRadix : 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (total) n = usable_entries(total, capacity);
    const uint32_t base = blockIdx.x * kTileKeys;
    if (base >= n) return;  // whole workgroup
    s_hist[tid] = 0;
    if (TT) s_tt[tid] = 0;
    __syncthreads();
    const uint32_t seg = base + wave * (64 * ITEMS);
    K key[ITEMS];
    uint32_t tt[ITEMS];
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const uint32_t pos = seg + i * 64 + lane;
        key[i] = pos < n ? keys[pos] : K(0);
        tt[i] = TT && pos < n ? tiles_touched[vals[pos]] : 0u;
    }
#pragma unroll
    for (int i = 0; i < ITEMS; ++i) {
        const bool valid = seg + i * 64 + lane < n;
        const uint32_t d = digit_of(key[i], shift);
        const uint64_t peers = match_digit(d, valid);
        if (valid && lane == __ffsll((unsigned long long)peers) - 1)
            atomicAdd(&s_hist[d], (uint32_t)__popcll(peers));
        if (TT && valid && tt[i] != 0u) atomicAdd(&s_tt[d], tt[i]);
    }
    __syncthreads();
    emit_counts(s_hist, (int)gridDim.x, counts);
    if (TT) emit_counts(s_tt, (int)gridDim.x, tt_counts);
}

// One pass's 256 rows of per-tile digit counts (row d at counts + d *
// stride): hist[d] = the total of the row's first nblk tiles, and the row is
// replaced in place by its exclusive prefix over tiles. nblk covers the
// usable entries (*total, capacity) when total is given. One workgroup of
// kScanThreads per row, each thread a run of consecutive tiles (a row can
// be tens of thousands of tiles long when many views are binned at once).
// If tt_counts is given (the last depth pass), its rows are scanned the same
// way in 64 bits into tt_prefix, with totals in tt_hist.
constexpr int kScanThreads = 1024;
__global__ __launch_bounds__(kScanThreads) void k_count_scan(uint32_t* __restrict__ counts, int stride, int nblk,
                                                             const uint64_t* __restrict__ total, uint32_t capacity,
                                                             int tile_keys, uint32_t* __restrict__ hist,
                                                             const uint32_t* __restrict__ tt_counts,
                                                             uint64_t* __restrict__ tt_prefix,
                                                             uint64_t* __restrict__ tt_hist) {
    constexpr int kWaves = kScanThreads / 64;
    __shared__ uint32_t s_w[kWaves];
    __shared__ uint64_t s_w64[kWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = blockIdx.x;
    if (total) nblk = (int)((usable_entries(total, capacity) + (uint32_t)tile_keys - 1) / (uint32_t)tile_keys);
    uint32_t* row = counts + (size_t)r * stride;
    const int per = (nblk + kScanThreads - 1) / kScanThreads;
    const int i0 = min(tid * per, nblk), i1 = min(i0 + per, nblk);
    uint32_t sum = 0;
    for (int i = i0; i < i1; ++i) sum += row[i];
    uint32_t incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)incl, off, 64);
        if (lane >= off) incl += y;
    }
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    uint32_t pre = 0, row_total = 0;
    for (int w = 0; w < kWaves; ++w) {
        const uint32_t x = s_w[w];
        pre += w < wave ? x : 0u;
        row_total += x;
    }
    uint32_t run = pre + incl - sum;
    for (int i = i0; i < i1; ++i) {
        const uint32_t c = row[i];
        row[i] = run;
        run += c;
    }
    if (tid == 0) hist[r] = row_total;
    if (tt_counts) {
        const uint32_t* trow = tt_counts + (size_t)r * stride;
        uint64_t* prow = tt_prefix + (size_t)r * stride;
        uint64_t tsum = 0;
        for (int i = i0; i < i1; ++i) tsum += trow[i];
        uint64_t tincl = tsum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint64_t y = shfl_up_u64(tincl, off);
            if (lane >= off) tincl += y;
        }
        if (lane == 63) s_w64[wave] = tincl;
        __syncthreads();
        uint64_t tpre = 0, ttot = 0;
        for (int w = 0; w < kWaves; ++w) {
            const uint64_t x = s_w64[w];
            tpre += w < wave ? x : 0ull;
            ttot += x;
        }
        uint64_t trun = tpre + tincl - tsum;
        for (int i = i0; i < i1; ++i) {
            prow[i] = trun;
            trun += trow[i];
        }
        if (tid == 0) tt_hist[r] = ttot;
    }
}

// One stable radix pass over n (key, value) pairs on digit (key >> shift),
// 256 * ITEMS keys per workgroup (tile b = workgroup b).
//   hist         [256] digit totals of this pass
//   prefix       [256][nblk] per-tile exclusive prefix of each digit
// The key count is n, or the usable entries (*total, capacity) when total
// is given (the grid is then sized for the capacity; idle workgroups exit).
//
// With TT (the last depth pass, whose output order is the depth order) the
// pass also does the exclusive scan of tiles_touched in that order: the sum
// over the splats before position `out` is the sum over all smaller digits
// (exclusive scan of tt_hist), over this digit in earlier tiles (tt_prefix)
// and over this digit earlier in this tile (a scan of the staged slots). It
// writes offsets[out], first_owner[B] for every duplication workgroup B
// whose first entry the splat owns, and the entry count E to *tt_total_out
// (and *n_dev if given).
struct DepthScanArgs {
    const uint32_t* tiles_touched;
    const uint64_t* tt_prefix;  // [256][nblk]
    const uint64_t* tt_hist;    // [256]
    uint32_t* offsets;
    uint32_t* first_owner;
    uint32_t n_dup_blocks;
    uint64_t* tt_total_out;
    uint64_t* n_dev;
};

template <typename K, int ITEMS, bool TT>
__global__ __launch_bounds__(kSortThreads) void k_radix_pass(
    const K* __restrict__ keys_in, const uint32_t* __restrict__ vals_in, uint32_t n,
    const uint64_t* __restrict__ total, uint32_t capacity, int shift, const uint32_t* __restrict__ hist,
    const uint32_t* __restrict__ prefix, K* __restrict__ keys_out, uint32_t* __restrict__ vals_out,
    DepthScanArgs ds) {
    constexpr int kTileKeys = kSortThreads * ITEMS;
    __shared__ uint32_t s_wcount[kSortWaves][kRadix];  // per-wave digit counts, then prefixes
    __shared__ uint32_t s_local_start[kRadix];
    __shared__ uint32_t s_gbase[kRadix];
    __shared__ uint32_t s_wsum[3][4];
    __shared__ K s_keys[kTileKeys];
    __shared__ uint32_t s_vals[kTileKeys];
    __shared__ uint32_t s_tt[TT ? kTileKeys : 1];   // tiles_touched per staged slot
    __shared__ uint32_t s_ttx[TT ? kTileKeys : 1];  // its exclusive scan over the slots
    __shared__ uint64_t s_ttbase[TT ? kRadix : 1];
    __shared__ uint64_t s_wsum64[4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t b = blockIdx.x;
    const uint32_t base = b * kTileKeys;
    if (total) n = usable_entries(total, capacity);
    if (base >= n) return;  // whole workgroup
#pragma unroll
    for (int w = 0; w < kSortWaves; ++w) s_wcount[w][tid] = 0;
    __syncthreads();

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

    const uint32_t excl = prefix[(size_t)d * gridDim.x + b];
    s_gbase[d] = dstart + excl;
    if (TT) {
        const uint64_t th = ds.tt_hist[d];
        const uint64_t tstart = block_exclusive_scan_u64(th, s_wsum64);
        s_ttbase[d] = tstart + ds.tt_prefix[(size_t)d * gridDim.x + b];
        if (b == 0 && d == kRadix - 1) {
            *ds.tt_total_out = tstart + th;
            if (ds.n_dev) *ds.n_dev = tstart + th;
        }
    }
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
            if (TT) s_tt[slot] = ds.tiles_touched[val[i]];
        }
    }
    __syncthreads();
    const uint32_t valid_n = min(n - base, (uint32_t)kTileKeys);
    if (TT) {  // exclusive scan of s_tt over the slots (thread t: slots [ITEMS t, ITEMS t + ITEMS))
        uint32_t c[ITEMS];
        uint32_t sum = 0;
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            const uint32_t sl = tid * ITEMS + j;
            c[j] = sl < valid_n ? s_tt[sl] : 0u;
            sum += c[j];
        }
        uint32_t run = block_exclusive_scan_fast(sum, s_wsum[2]);
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            s_ttx[tid * ITEMS + j] = run;
            run += c[j];
        }
        __syncthreads();
    }
    for (uint32_t s = tid; s < valid_n; s += kSortThreads) {
        const K k = s_keys[s];
        const uint32_t dd = digit_of(k, shift);
        const uint32_t out = s_gbase[dd] + (s - s_local_start[dd]);
        keys_out[out] = k;
        vals_out[out] = s_vals[s];
        if (TT) {
            const uint64_t off = s_ttbase[dd] + (s_ttx[s] - s_ttx[s_local_start[dd]]);
            const uint32_t cnt = s_tt[s];
            ds.offsets[out] = (uint32_t)off;
            if (cnt != 0u) {  // duplication workgroups whose first entry this splat owns
                const uint64_t b1 = (off + cnt - 1) / kDupTile;
                for (uint64_t B = (off + kDupTile - 1) / kDupTile; B <= b1 && B < ds.n_dup_blocks; ++B)
                    ds.first_owner[B] = out;
            }
        }
    }
}

// ---- tile ranges ----

__global__ void k_fill_u32(uint32_t* __restrict__ p, size_t n, uint32_t v) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// Every tile's range from the sorted tile ids: a run's first entry writes
// its start, its last entry its end; the tiles between two runs, before the
// first and after the last get (0, 0). Each lane that ends a run (and the
// first entry, for the tiles before it) names the gap of empty tiles that
// follows, and its wave clears every such gap 64 tiles at a time. With at
// least one entry every tile of the n_tiles is written; with none,
// k_tile_schedule clears them. The count is n, or the usable entries
// (*total, capacity) when total is given.
__global__ void k_ranges(const uint64_t* __restrict__ keys, uint32_t n, const uint64_t* __restrict__ total,
                         uint32_t capacity, uint32_t n_tiles, uint32_t* __restrict__ ranges) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    const int lane = threadIdx.x & 63;
    // The tile ids (high words) of entries i - 1, i and i + 1, loaded at once
    // and before the entry count is known, within the keys buffer (capacity
    // entries when the count comes from the device, else n); entries at or
    // past the count are not used.
    const uint32_t bound = total ? capacity : n;
    const uint32_t* const khi = reinterpret_cast<const uint32_t*>(keys) + 1;
    uint32_t tp = 0, t = 0, tn = 0;
    if (i < bound) {
        tp = khi[2 * (size_t)(i > 0 ? i - 1 : 0)];
        t = khi[2 * (size_t)i];
        tn = khi[2 * (size_t)(i + 1 < bound ? i + 1 : i)];
    }
    if (total) n = usable_entries(total, capacity);
    uint2* const r2 = reinterpret_cast<uint2*>(ranges);
    uint32_t g0 = 0, g1 = 0, h1 = 0;  // empty tiles [g0, g1) after this run; [0, h1) before the first
    if (i < n) {
        if (i == 0) h1 = min(t, n_tiles);
        if (i == 0 || tp != t) ranges[2 * (size_t)t] = i;
        const uint32_t next = i == n - 1 ? n_tiles : tn;
        if (next != t) {
            ranges[2 * (size_t)t + 1] = i + 1;
            g0 = t + 1;
            g1 = min(next, n_tiles);
        }
    }
    // the whole wave clears each named gap (every lane takes part, in range or not)
    for (int pass = 0; pass < 2; ++pass) {
        const uint32_t lo = pass ? g0 : 0u, hi = pass ? g1 : h1;
        uint64_t m = __ballot(hi > lo);
        while (m) {
            const int l = __ffsll((unsigned long long)m) - 1;
            m &= m - 1;
            const uint32_t a = (uint32_t)__shfl((int)lo, l, 64), b = (uint32_t)__shfl((int)hi, l, 64);
            for (uint32_t u = a + (uint32_t)lane; u < b; u += 64) r2[u] = make_uint2(0u, 0u);
        }
    }
}

// Sort class of a tile for heaviest-first scheduling: 255 - (1 + 16 log2
// of its list length, 16 linear steps per octave), clamped; empty tiles last.
__device__ __forceinline__ uint32_t heavy_first_key(uint32_t len) {
    if (len == 0u) return 255u;
    const int msb = 31 - __clz((int)len);
    const uint32_t frac = ((len << (31 - msb)) >> 27) & 15u;  // the 4 bits below the leading one
    return 255u - min(255u, 1u + 16u * (uint32_t)msb + frac);
}

// The compositing schedules, from ranges that k_ranges wrote for every
// tile; with no usable entries (E = 0, or E > capacity), when k_ranges
// wrote nothing, every range is set to (0, 0) here instead.
// order = the tiles in descending order of list length (by class; the
// order within a class is unspecified). chunks = the work items of the
// scheduled compositing after a count (padded to 16 bytes), each (tile,
// chunk index, list start, list length). When the lists average more than
// one chunk (E > kChunk tiles), every list longer than a chunk is cut into
// kChunk-entry chunks and shorter ones (empty ones too) are whole items
// (chunk index kWholeList); otherwise every list is a whole item. Items
// come in descending order of the list length from the item's start to the
// list's end: the front chunks of the longest lists first, since a pixel
// that stops early leaves the later chunks of its list little to do. order
// and chunks may be NULL.
//
// One workgroup of 1024 threads, each over the same kSweep tiles per sweep
// in both passes: class histograms, exclusive scans, then placement through
// per-class cursors. Empty tiles, often the largest class, go last in the
// order of a block scan of per-thread counts. (Bumping the LDS counters once
// per run of equal classes in a wave, or spreading the work over several
// workgroups that each count every tile, measured slower.)
constexpr int kOrderThreads = 1024;

__global__ __launch_bounds__(kOrderThreads) void k_tile_schedule(uint32_t* __restrict__ ranges, int n_tiles,
                                                                 const uint64_t* __restrict__ total,
                                                                 uint32_t n_entries, uint32_t capacity,
                                                                 uint32_t* __restrict__ order,
                                                                 uint32_t* __restrict__ chunks) {
    constexpr int kSweep = 8;                             // tiles per thread per sweep, loaded together
    constexpr int kSweepTiles = kOrderThreads * kSweep;
    __shared__ uint32_t s_hist[2][kRadix];  // non-empty tiles, their chunk items per class; then the cursors
    __shared__ uint32_t s_wsum[2][kRadix / 64];
    __shared__ uint32_t s_esum[kOrderThreads / 64];
    __shared__ uint32_t s_items[2];  // non-empty tiles, their items
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint2* const r2 = reinterpret_cast<uint2*>(ranges);
    const uint32_t E = total ? usable_entries(total, capacity) : n_entries;
    // lists longer than `cut` become chunks: every list of more than a chunk
    // when the lists average more than one, else none (the tiles alone then
    // give a compositing launch enough workgroups; cutting the longest lists
    // too measured slower)
    const uint32_t cut = (uint64_t)E > (uint64_t)kChunk * (uint64_t)n_tiles ? (uint32_t)kChunk : 0xFFFFFFFFu;
    const bool split = chunks != nullptr;  // the items, by the classes of the chunks
    const bool by_tile = order != nullptr;  // the tile classes
    const bool sched = order || chunks;
    uint4* const items = chunks ? reinterpret_cast<uint4*>(chunks + 4) : nullptr;
    if (tid < 2 * kRadix) (&s_hist[0][0])[tid] = 0u;
    __syncthreads();
    // 1. check every range; count the classes of the non-empty tiles and of
    //    their chunk items, and this thread's empty tiles
    uint2 r[kSweep];
    uint32_t empties = 0;
    for (int base = 0; base < n_tiles; base += kSweepTiles) {
        if (E > 0u) {  // (E is uniform) the sweep's ranges in one batch of loads
#pragma unroll
            for (int k = 0; k < kSweep; ++k) {
                const int t = base + k * kOrderThreads + tid;
                r[k] = t < n_tiles ? r2[t] : make_uint2(0u, 0u);
            }
        } else {  // no usable entries: every range becomes (0, 0)
#pragma unroll
            for (int k = 0; k < kSweep; ++k) {
                const int t = base + k * kOrderThreads + tid;
                r[k] = make_uint2(0u, 0u);
                if (t < n_tiles) r2[t] = r[k];
            }
        }
        if (!sched) continue;
#pragma unroll
        for (int k = 0; k < kSweep; ++k) {
            const int t = base + k * kOrderThreads + tid;
            const uint32_t len = r[k].y - r[k].x;
            if (t >= n_tiles) continue;
            if (len == 0u) {
                ++empties;
                continue;
            }
            if (by_tile) atomicAdd(&s_hist[0][heavy_first_key(len)], 1u);
            if (split) {
                // a list up to the cut length is one item; a longer one has
                // one per chunk, classed by the length from the chunk on
                if (len <= cut)
                    atomicAdd(&s_hist[1][heavy_first_key(len)], 1u);
                else
                    for (uint32_t at = 0; at < len; at += kChunk) atomicAdd(&s_hist[1][heavy_first_key(len - at)], 1u);
            }
        }
    }
    if (!sched) return;
    __syncthreads();  // every count of step 1 is in
    // 2. class starts (exclusive scans); the empty tiles follow all others in
    //    the order of an exclusive block scan of the per-thread counts
    uint32_t einc = empties;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)einc, off, 64);
        if (lane >= off) einc += y;
    }
    if (lane == 63) s_esum[wave] = einc;
    const int which = tid >> 8, cls = tid & (kRadix - 1), w4 = (tid >> 6) & 3;
    uint32_t h = 0, incl = 0;
    if (tid < 2 * kRadix) {
        h = s_hist[which][cls];
        incl = h;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const uint32_t y = (uint32_t)__shfl_up((int)incl, off, 64);
            if (lane >= off) incl += y;
        }
        if (lane == 63) s_wsum[which][w4] = incl;
    }
    __syncthreads();
    uint32_t erank = einc - empties, etot = 0;  // this thread's first empty tile among the empty ones
    for (int w = 0; w < kOrderThreads / 64; ++w) {
        erank += w < wave ? s_esum[w] : 0u;
        etot += s_esum[w];
    }
    if (tid < 2 * kRadix) {
        uint32_t pre = 0, all = 0;
        for (int w = 0; w < 4; ++w) {
            pre += w < w4 ? s_wsum[which][w] : 0u;
            all += s_wsum[which][w];
        }
        s_hist[which][cls] = pre + incl - h;  // now the class cursors
        if (cls == 0) s_items[which] = all;
    }
    __syncthreads();
    // the empty tiles come after every other tile and item
    const uint32_t filled_tiles = (uint32_t)n_tiles - etot, filled_items = split ? s_items[1] : filled_tiles;
    // 3. placement (a single sweep keeps its checked ranges in registers).
    //    Positions stay below the tile count and the schedule's length by
    //    construction; the guards keep a write inside the buffers regardless.
    const uint32_t max_items = (uint32_t)n_tiles + (capacity + (uint32_t)kChunk - 1u) / (uint32_t)kChunk;
    auto put_order = [&](uint32_t pos, uint32_t t) {
        if (order && pos < (uint32_t)n_tiles) order[pos] = t;
    };
    auto put_item = [&](uint32_t pos, uint4 it) {
        if (pos < max_items) items[pos] = it;
    };
    for (int base = 0; base < n_tiles; base += kSweepTiles) {
        if (n_tiles > kSweepTiles) {
#pragma unroll
            for (int k = 0; k < kSweep; ++k) {
                const int t = base + k * kOrderThreads + tid;
                r[k] = t < n_tiles && E > 0u ? r2[t] : make_uint2(0u, 0u);
            }
        }
#pragma unroll
        for (int k = 0; k < kSweep; ++k) {
            const int t = base + k * kOrderThreads + tid;
            if (t >= n_tiles) continue;
            const uint32_t start = r[k].x, len = r[k].y - r[k].x;
            if (len == 0u) {
                const uint32_t rank = erank++;
                put_order(filled_tiles + rank, (uint32_t)t);
                if (chunks) put_item(filled_items + rank, make_uint4((uint32_t)t, kWholeList, 0u, 0u));
                continue;
            }
            if (by_tile) put_order(atomicAdd(&s_hist[0][heavy_first_key(len)], 1u), (uint32_t)t);
            if (split) {
                if (len <= cut)
                    put_item(atomicAdd(&s_hist[1][heavy_first_key(len)], 1u),
                             make_uint4((uint32_t)t, kWholeList, start, len));
                else
                    for (uint32_t at = 0, b = 0; at < len; at += kChunk, ++b)
                        put_item(atomicAdd(&s_hist[1][heavy_first_key(len - at)], 1u),
                                 make_uint4((uint32_t)t, b, start, len));
            }
        }
    }
    // the item count: every chunk item and empty list, or every tile
    if (chunks && tid == 0) chunks[0] = filled_items + etot;
}

int tile_pass_count(int tile_bits) { return (tile_bits + 7) / 8; }

}  // namespace

size_t bin_scratch_layout(int n, int64_t capacity, BinScratch* out, void* base) {
    const size_t nb_gauss = (size_t)(n + kGaussTile - 1) / kGaussTile;
    const size_t nb_entry = (size_t)((capacity + kEntryTile - 1) / kEntryTile);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align256(bytes > 0 ? bytes : 1);
        return at;
    };
    const size_t o_tot = take(8);
    const size_t o_ghist = take((size_t)kGaussPasses * kRadix * 4);
    const size_t o_ehist = take((size_t)kMaxTilePasses * kRadix * 4);
    const size_t o_gcnt = take(nb_gauss * kRadix * kGaussPasses * 4);
    const size_t o_ecnt = take(nb_entry * kRadix * kMaxTilePasses * 4);
    const size_t o_ttc = take(nb_gauss * kRadix * 4);
    const size_t o_ttp = take(nb_gauss * kRadix * 8);
    const size_t o_tth = take(kRadix * 8);
    const size_t o_off = take((size_t)n * 4);
    const size_t o_fo = take(nb_entry * 4);
    const size_t o_gk0 = take((size_t)n * 4);
    const size_t o_gv0 = take((size_t)n * 4);
    const size_t o_gk1 = take((size_t)n * 4);
    const size_t o_gv1 = take((size_t)n * 4);
    const size_t o_kt = take((size_t)capacity * 8);
    const size_t o_vt = take((size_t)capacity * 4);
    if (out && base) {
        char* b = (char*)base;
        out->total = (uint64_t*)(b + o_tot);
        out->gauss_hist = (uint32_t*)(b + o_ghist);
        out->entry_hist = (uint32_t*)(b + o_ehist);
        out->gauss_counts = (uint32_t*)(b + o_gcnt);
        out->entry_counts = (uint32_t*)(b + o_ecnt);
        out->tt_counts = (uint32_t*)(b + o_ttc);
        out->tt_prefix = (uint64_t*)(b + o_ttp);
        out->tt_hist = (uint64_t*)(b + o_tth);
        out->offsets = (uint32_t*)(b + o_off);
        out->first_owner = (uint32_t*)(b + o_fo);
        out->gk[0] = (uint32_t*)(b + o_gk0);
        out->gv[0] = (uint32_t*)(b + o_gv0);
        out->gk[1] = (uint32_t*)(b + o_gk1);
        out->gv[1] = (uint32_t*)(b + o_gv1);
        out->keys_tmp = (uint64_t*)(b + o_kt);
        out->vals_tmp = (uint32_t*)(b + o_vt);
    }
    return off;
}

// The stable depth order of the n splats (culled last) into s.gv[0], with
// the scan of their tile counts in that order riding on the last pass
// (offsets, first_owner, E to s.total and *n_dev), ITEMS keys per lane.
template <int ITEMS>
void launch_depth_sort(int n, const float4* xy_depth, const uint32_t* tiles_touched, const BinScratch& s,
                       unsigned nbe, uint64_t* n_dev, hipStream_t stream) {
    const unsigned nbg = (unsigned)((n + kSortThreads * ITEMS - 1) / (kSortThreads * ITEMS));
    hipLaunchKernelGGL(k_depth_keys<ITEMS>, dim3(nbg), dim3(kSortThreads), 0, stream, xy_depth, tiles_touched, n,
                       s.gk[0], s.gv[0], s.gauss_counts);
    const DepthScanArgs none{};
    const DepthScanArgs scan{tiles_touched, s.tt_prefix, s.tt_hist, s.offsets, s.first_owner, nbe, s.total, n_dev};
    for (int p = 0; p < kGaussPasses; ++p) {
        const int src = p & 1, dst = src ^ 1;  // an even pass count leaves the order in gv[0]
        const bool last = p == kGaussPasses - 1;
        uint32_t* cnt = s.gauss_counts + (size_t)p * kRadix * nbg;
        if (last)
            hipLaunchKernelGGL((k_count_digits<uint32_t, ITEMS, true>), dim3(nbg), dim3(kSortThreads), 0,
                               stream, s.gk[src], (uint32_t)n, (const uint64_t*)nullptr, 0u, 8 * p, cnt,
                               (const uint32_t*)s.gv[src], tiles_touched, s.tt_counts);
        else if (p > 0)
            hipLaunchKernelGGL((k_count_digits<uint32_t, ITEMS, false>), dim3(nbg), dim3(kSortThreads), 0,
                               stream, s.gk[src], (uint32_t)n, (const uint64_t*)nullptr, 0u, 8 * p, cnt,
                               (const uint32_t*)nullptr, (const uint32_t*)nullptr, (uint32_t*)nullptr);
        hipLaunchKernelGGL(k_count_scan, dim3(kRadix), dim3(kScanThreads), 0, stream, cnt, (int)nbg, (int)nbg,
                           (const uint64_t*)nullptr, 0u, kSortThreads * ITEMS, s.gauss_hist + p * kRadix,
                           last ? (const uint32_t*)s.tt_counts : nullptr, last ? s.tt_prefix : nullptr,
                           last ? s.tt_hist : nullptr);
        if (last)
            hipLaunchKernelGGL((k_radix_pass<uint32_t, ITEMS, true>), dim3(nbg), dim3(kSortThreads), 0,
                               stream, s.gk[src], s.gv[src], (uint32_t)n, (const uint64_t*)nullptr, 0u, 8 * p,
                               s.gauss_hist + p * kRadix, cnt, s.gk[dst], s.gv[dst], scan);
        else
            hipLaunchKernelGGL((k_radix_pass<uint32_t, ITEMS, false>), dim3(nbg), dim3(kSortThreads), 0,
                               stream, s.gk[src], s.gv[src], (uint32_t)n, (const uint64_t*)nullptr, 0u, 8 * p,
                               s.gauss_hist + p * kRadix, cnt, s.gk[dst], s.gv[dst], none);
    }
}

hipError_t launch_bin_and_sort(const gs_camera& cam, int n_views, int n, const float4* xy_depth,
                               const float4* conic_op, const uint32_t* tiles_touched, uint64_t* keys,
                               uint32_t* values, uint32_t capacity, const BinScratch& s, uint64_t* n_dev,
                               uint32_t flags, hipStream_t stream) {
    // 1. stable depth order of the splats (culled last) into gv[0]; the last
    // pass also scans tiles_touched in that order: offsets, first_owner, E
    const unsigned nbe = (capacity + kEntryTile - 1) / kEntryTile;
    if (n >= kGaussBigN)
        launch_depth_sort<kGaussItemsBig>(n, xy_depth, tiles_touched, s, nbe, n_dev, stream);
    else
        launch_depth_sort<kGaussItems>(n, xy_depth, tiles_touched, s, nbe, n_dev, stream);
    // 2. duplication and the stable sort on the tile-id bits. Grids cover the
    // capacity; the kernels read E and do nothing when it exceeds capacity.
    if (nbe == 0) return hipGetLastError();
    int tile_bits = 0;
    while ((int64_t)1 << tile_bits < (int64_t)tiles_x(cam) * tiles_y(cam) * n_views) ++tile_bits;
    const uint32_t n_view = (uint32_t)max(1, n / n_views);  // splats per view (n_views divides n)
    const int passes = tile_pass_count(tile_bits);
    // the tile bits split evenly over the passes (e.g. 7 + 6 for 13 bits):
    // with fewer digit values per pass each workgroup scatters longer runs
    // per digit (measured against 8 + 5: binning -0.8 us at 1080p/160k,
    // -4.3 us at 1080p/1M)
    int pass_arg[4];
    for (int p = 0, lo = 0; p < passes; ++p) {
        const int width = (tile_bits - lo + (passes - p) - 1) / (passes - p);
        pass_arg[p] = digit_pass(32 + lo, width);
        lo += width;
    }
    // entries start in the tmp pair when the pass count is odd, so the last
    // pass always writes (keys, values)
    uint64_t* kin = (passes & 1) ? s.keys_tmp : keys;
    uint32_t* vin = (passes & 1) ? s.vals_tmp : values;
    uint64_t* kout = (passes & 1) ? keys : s.keys_tmp;
    uint32_t* vout = (passes & 1) ? values : s.vals_tmp;
    if (flags & kTilesEllipse)
        hipLaunchKernelGGL(k_duplicate<true>, dim3(nbe), dim3(kDupThreads), 0, stream, xy_depth, conic_op,
                           s.offsets, s.gv[0], s.first_owner, n, (const uint64_t*)s.total, capacity, tiles_x(cam),
                           tiles_y(cam), n_view, passes, passes > 0 ? pass_arg[0] : 0, kin, vin, s.entry_counts);
    else
        hipLaunchKernelGGL(k_duplicate<false>, dim3(nbe), dim3(kDupThreads), 0, stream, xy_depth, conic_op,
                           s.offsets, s.gv[0], s.first_owner, n, (const uint64_t*)s.total, capacity, tiles_x(cam),
                           tiles_y(cam), n_view, passes, passes > 0 ? pass_arg[0] : 0, kin, vin, s.entry_counts);
    for (int p = 0; p < passes; ++p) {
        uint32_t* cnt = s.entry_counts + (size_t)p * kRadix * nbe;
        if (p > 0)
            hipLaunchKernelGGL((k_count_digits<uint64_t, kEntryItems, false>), dim3(nbe), dim3(kSortThreads), 0,
                               stream, kin, 0u, (const uint64_t*)s.total, capacity, pass_arg[p], cnt,
                               (const uint32_t*)nullptr, (const uint32_t*)nullptr, (uint32_t*)nullptr);
        hipLaunchKernelGGL(k_count_scan, dim3(kRadix), dim3(kScanThreads), 0, stream, cnt, (int)nbe, 0,
                           (const uint64_t*)s.total, capacity, kEntryTile, s.entry_hist + p * kRadix,
                           (const uint32_t*)nullptr, (uint64_t*)nullptr, (uint64_t*)nullptr);
        hipLaunchKernelGGL((k_radix_pass<uint64_t, kEntryItems, false>), dim3(nbe), dim3(kSortThreads), 0, stream,
                           kin, vin, 0u, (const uint64_t*)s.total, capacity, pass_arg[p], s.entry_hist + p * kRadix,
                           cnt, kout, vout, DepthScanArgs{});
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
                              int n_tiles, uint32_t* ranges, uint32_t* tile_order, uint32_t* chunks,
                              hipStream_t stream) {
    // mark the run boundaries, then check every tile's range against the keys
    // (empty tiles become (0, 0)) and build the schedules
    const uint32_t grid_n = n_dev ? capacity : n_entries;
    if (grid_n > 0)
        hipLaunchKernelGGL(k_ranges, dim3((grid_n + 255) / 256), dim3(256), 0, stream, keys, n_entries, n_dev,
                           capacity, (uint32_t)n_tiles, ranges);
    if (n_tiles > 0)
        hipLaunchKernelGGL(k_tile_schedule, dim3(1), dim3(kOrderThreads), 0, stream, ranges, n_tiles, n_dev,
                           n_entries, capacity, tile_order, chunks);
    return hipGetLastError();
}

}  // namespace gs
