// Stable counting sort of token indices by bucket id: the block-sparse layout
// that bucket attention gathers from (FAST-AR summary, "2. Core Components",
// part C).  Two launches, every count stays on the device:
//
//   sort_hist    one block per 1024-id tile: LDS histogram -> hist[h][tile][b]
//   sort_scatter one block per tile: first the tile's base offsets, from the
//                histograms of all tiles of its head (ids below b anywhere,
//                plus ids equal to b in earlier tiles); block 0 of each head
//                also writes off[h][b].  Then the stable rank of every id
//                inside its tile (wave ballots on the P id bits give the rank
//                among equal ids of the wave; LDS counters tagged by round
//                carry it across waves and rounds), and perm[base + rank] =
//                index (from kSortStagedTiles tiles per head on, the tile's
//                indices go through LDS in bucket order first, so that the
//                stores form runs).  For a (queries, keys) pair of sets one more block
//                per head builds the attention work list (one item per bucket
//                and 64- or 256-query slice, longest key lists first) beside the
//                tiles.  The tile's ids are loaded before the histograms, so
//                both loads are in flight together.
//
// Every block re-reads its head's tile histograms (a few KB, from L2) instead
// of waiting for a separate scan launch -- up to kSortScanTiles tiles per head;
// beyond that a scan launch (one block per head and set) turns the
// histograms into per-tile prefixes first.  The result is unique (a stable sort),
// so it is bit-identical run to run.
#include "common.hpp"
#include "launch.hpp"

namespace fastar {

// Up to kSortMaxSets sets in one launch (grid z / y = set).  With work lists
// the sets come in (queries, keys) pairs 2p, 2p+1, and pair p's list goes to
// items[p] (multi-table AnnSA sorts every table's pair at once).
struct SortArgs {
    IdSet set[kSortMaxSets];
    SortBufs buf[kSortMaxSets];
    ItemTable items[kSortMaxPairs];
    int nsets;
    int npairs;                   // pairs with a work list (then nsets = 2 * npairs)
    int B;
    int P;
    int builder_block;            // grid x index of the work-list blocks, or -1
    int scanned;                  // hist holds per-tile prefixes and off is written (scan launch)
    int staged;                   // perm written from LDS in bucket order (coalesced runs)
};

__device__ __forceinline__ int set_count(const IdSet& s, int h, int& na) {
    na = s.a_nvalid ? clamp_n(s.a_nvalid, h, s.a_cap) : s.a_fixed;
    return na + s.nb;
}

// The bucket of element min(e, n - 1) of a set with n >= 1 elements, read
// with no branch (the row pointer is selected, then loaded): loads under a
// branch each get their own wait, so a thread's loads would run one after
// another instead of all in flight together.
__device__ __forceinline__ int set_bucket(const IdSet& s, int h, int na, int n, int e, int B) {
    e = min(e, n - 1);
    const uint16_t* pa = s.a + static_cast<size_t>(h) * s.a_stride + e;
    const uint16_t* pb = s.b + static_cast<size_t>(h) * s.b_stride + (e - na);
    return (*(e < na ? pa : pb) >> s.shift) & (B - 1);
}

__global__ __launch_bounds__(256) void sort_hist_kernel(SortArgs a) {
    __shared__ int cnt[1024];
    const IdSet& S = a.set[blockIdx.z];
    const SortBufs& O = a.buf[blockIdx.z];
    const int h = blockIdx.y, t = blockIdx.x, B = a.B;
    int na;
    const int n = set_count(S, h, na);
    if (t * kSortTile >= n) return;
    constexpr int R = kSortTile / 256;
    int id[R];
#pragma unroll
    for (int r = 0; r < R; ++r) id[r] = set_bucket(S, h, na, n, t * kSortTile + r * 256 + threadIdx.x, B);
    for (int b = threadIdx.x; b < B; b += 256) cnt[b] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r)
        if (t * kSortTile + r * 256 + static_cast<int>(threadIdx.x) < n) atomicAdd(&cnt[id[r]], 1);
    __syncthreads();
    int* dst = O.hist + (static_cast<size_t>(h) * O.max_tiles + t) * B;
    for (int b = threadIdx.x; b < B; b += 256) dst[b] = cnt[b];
}

// Per-bucket sums of one set's tile counts -- over the tiles before ``t`` and
// over all tiles -- for the buckets of this thread.  With B <= 256 every
// bucket b is summed by 256 / B threads (part p, b), each over a contiguous
// range of tiles whose counts it loads in one go (up to kTileLoads at once);
// the parts meet in LDS and thread b keeps bucket b (k = 1).  With B > 256
// thread i keeps buckets i*k .. i*k+k-1 (k = B / 256) and sums all tiles.
constexpr int kTileLoads = 32;
// Keys per tile of the attention kernels: an item's cost is its key tiles,
// which order the work list (only the order, never a result, depends on it).
constexpr int kItemKeyTile = 64;
// Tiles per head above which the histograms are scanned in a launch of their
// own.  Measured over 12 heads of 128 buckets: at 75 tiles the two-launch
// form takes 21.9 us and the three-launch form 27.8; at 293 tiles 77 and
// 57.8.  (The step's 37 tiles keep the two-launch form.)
constexpr int kSortScanTiles = 128;
// Tiles per head from which the scatter writes perm from LDS in bucket order
// (coalesced runs: a third fewer bytes written at 293 tiles, at the same
// time); at 74 tiles the extra scan and barriers cost 2 us of latency.
#ifndef SORT_STAGED_TILES
#define SORT_STAGED_TILES 128
#endif
constexpr int kSortStagedTiles = SORT_STAGED_TILES;

struct BucketSums {
    int before[4], total[4];
};

__device__ __forceinline__ void bucket_sums(const SortBufs& O, int h, int t, int ntiles, int B, int k,
                                            BucketSums& s, int* pt, int* pb) {
    const int tid = threadIdx.x;
    const int* hh = O.hist + static_cast<size_t>(h) * O.max_tiles * B;
#pragma unroll
    for (int j = 0; j < 4; ++j) s.before[j] = s.total[j] = 0;
    if (k == 1) {
        const int parts = 256 / B, part = tid / B, b = tid % B;
        int sum = 0, bef = 0;
        if (part < parts) {
            const int tpp = (ntiles + parts - 1) / parts;
            const int t0 = min(ntiles, part * tpp), t1 = min(ntiles, t0 + tpp);
            for (int c0 = t0; c0 < t1; c0 += kTileLoads) {
                int c[kTileLoads];
#pragma unroll
                for (int i = 0; i < kTileLoads; ++i) c[i] = c0 + i < t1 ? hh[static_cast<size_t>(c0 + i) * B + b] : 0;
#pragma unroll
                for (int i = 0; i < kTileLoads; ++i) {
                    sum += c[i];
                    bef += c0 + i < t ? c[i] : 0;
                }
            }
            pt[part * B + b] = sum;
            pb[part * B + b] = bef;
        }
        __syncthreads();
        if (tid < B) {
            for (int q = 0; q < parts; ++q) {
                s.total[0] += pt[q * B + tid];
                s.before[0] += pb[q * B + tid];
            }
        }
        __syncthreads();                          // pt / pb may be reused
    } else {
        const int b0 = tid * k;
#pragma unroll 4
        for (int tt = 0; tt < ntiles; ++tt) {
            int c[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) c[j] = hh[static_cast<size_t>(tt) * B + b0 + min(j, k - 1)];   // no branch
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j < k) {
                    s.total[j] += c[j];
                    s.before[j] += tt < t ? c[j] : 0;
                }
            }
        }
    }
}

// Exclusive prefix over buckets (in bucket order) of the totals: ``start[j]``
// for the thread's buckets; returns the grand total.
__device__ __forceinline__ int bucket_starts(const BucketSums& s, int B, int k, int (&start)[4], int* smem) {
    const int b0 = threadIdx.x * k;
    int mine = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) mine += (j < k && b0 + j < B) ? s.total[j] : 0;
    int total;
    int run = block_exclusive_scan<256>(mine, smem, total);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        start[j] = run;
        run += (j < k && b0 + j < B) ? s.total[j] : 0;
    }
    return total;
}

// With many tiles per head (long key sets) the scatter blocks would each
// re-read every tile histogram of their head; one block per (head, set)
// instead turns the histograms into per-tile prefixes in place and writes
// off.  kScanNT threads: with B <= kScanNT each bucket's column is split into
// kScanNT / B contiguous tile ranges (parts); a part sums its range (loads in
// runs of kTileLoads), the parts' sums meet in LDS, and each part rewrites
// its range starting from the sum of the parts before it.  With B >
// kScanNT each thread walks whole columns.
constexpr int kScanNT = 1024;

__global__ __launch_bounds__(kScanNT) void sort_scan_kernel(SortArgs a) {
    __shared__ int smem[kScanNT / kWave];
    __shared__ int psum[kScanNT];
    const int h = blockIdx.x, si = blockIdx.y, B = a.B, tid = threadIdx.x;
    const IdSet& S = a.set[si];
    const SortBufs& O = a.buf[si];
    int na;
    const int ntiles = sort_tiles(set_count(S, h, na));
    int* hh = O.hist + static_cast<size_t>(h) * O.max_tiles * B;
    // thread -> (bucket, part): buckets fastest, so a load of one tile row is
    // coalesced over the buckets
    const int parts = B <= kScanNT ? kScanNT / B : 1;
    const int cols = B <= kScanNT ? 1 : B / kScanNT;        // columns per thread
    const int part = B <= kScanNT ? tid / B : 0;
    const int tpp = (ntiles + parts - 1) / parts;
    const int t0 = min(ntiles, part * tpp), t1 = min(ntiles, t0 + tpp);
    auto col_sum = [&](int b) {
        int sum = 0;
        for (int c0 = t0; c0 < t1; c0 += kTileLoads) {
            int c[kTileLoads];
#pragma unroll
            for (int i = 0; i < kTileLoads; ++i) c[i] = c0 + i < t1 ? hh[static_cast<size_t>(c0 + i) * B + b] : 0;
#pragma unroll
            for (int i = 0; i < kTileLoads; ++i) sum += c[i];
        }
        return sum;
    };
    auto col_rewrite = [&](int b, int running) {
        for (int c0 = t0; c0 < t1; c0 += kTileLoads) {
            int c[kTileLoads];
#pragma unroll
            for (int i = 0; i < kTileLoads; ++i) c[i] = c0 + i < t1 ? hh[static_cast<size_t>(c0 + i) * B + b] : 0;
#pragma unroll
            for (int i = 0; i < kTileLoads; ++i) {
                if (c0 + i < t1) hh[static_cast<size_t>(c0 + i) * B + b] = running;
                running += c[i];
            }
        }
        return running;
    };
    int mine = 0;                        // this thread's share of the bucket totals
    if (B <= kScanNT) {
        const int b = tid % B;
        const bool act = part < parts;
        const int sum = act ? col_sum(b) : 0;
        psum[tid] = sum;
        __syncthreads();
        int before = 0, total = 0;
        if (act) {
            for (int q = 0; q < parts; ++q) {
                const int v = psum[q * B + b];
                before += q < part ? v : 0;
                total += v;
            }
            col_rewrite(b, before);
        }
        mine = (act && part == 0) ? total : 0;
        __syncthreads();                 // psum is reused below only through smem
        int tot;
        const int run = block_exclusive_scan<kScanNT>(mine, smem, tot);
        int32_t* offp = O.off + static_cast<size_t>(h) * (B + 1);
        if (act && part == 0) offp[b] = run;
        if (tid == 0) offp[B] = tot;
    } else {
        int tots[4] = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (j < cols) tots[j] = col_rewrite(tid * cols + j, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) mine += tots[j];
        int tot;
        int run = block_exclusive_scan<kScanNT>(mine, smem, tot);
        int32_t* offp = O.off + static_cast<size_t>(h) * (B + 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < cols) offp[tid * cols + j] = run;
            run += tots[j];
        }
        if (tid == 0) offp[B] = tot;
    }
}

__global__ __launch_bounds__(256) void sort_scatter_kernel(SortArgs a) {
    __shared__ int run[1024];
    __shared__ int base[1024];
    __shared__ uint32_t wcnt[4][1024];
    __shared__ int smem[8];
    __shared__ int racc[256];
    const int si = blockIdx.z;
    const IdSet& S = a.set[si];
    const SortBufs& O = a.buf[si];
    const int h = blockIdx.y, t = blockIdx.x, B = a.B, P = a.P, tid = threadIdx.x;
    int na;
    const int n = set_count(S, h, na);
    const int ntiles = sort_tiles(n);
    const bool lead = t == 0;                     // writes off
    // the work-list builder: the extra last block of each query set's grid row
    const bool builder = a.npairs > 0 && t == a.builder_block;
    if (builder && (si & 1)) return;              // block uniform: key sets build nothing
    if (t >= ntiles && !lead && !builder) return; // block uniform
    const ItemTable& IT = a.items[builder ? si / 2 : 0];
    const IdSet& KSET = a.set[builder ? si + 1 : si];
    const SortBufs& KBUF = a.buf[builder ? si + 1 : si];
    const int k = (B + 255) / 256, b0 = tid * k;
    // the tile's ids, loaded first so their latency overlaps the histogram reads
    constexpr int R = kSortTile / 256;
    int idr[R];
    if (!builder && t < ntiles) {                 // block uniform
#pragma unroll
        for (int r = 0; r < R; ++r) idr[r] = set_bucket(S, h, na, n, t * kSortTile + r * 256 + tid, B);
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (t * kSortTile + r * 256 + tid >= n) idr[r] = 0;
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) idr[r] = 0;
    }

    // ---- the tile's base offsets (and, for the lead block, off); the part
    // sums borrow the rank step's LDS.  After a scan launch: off (bucket
    // starts) plus the tile's prefix, and the bucket totals from off.
    int* pt = reinterpret_cast<int*>(wcnt[0]);
    int* pb = reinterpret_cast<int*>(wcnt[1]);
    int32_t* offp = O.off ? O.off + static_cast<size_t>(h) * (B + 1) : nullptr;
    int start[4], tot[4];
    if (a.scanned) {
        const int* hh = O.hist + static_cast<size_t>(h) * O.max_tiles * B;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = b0 + j;
            start[j] = tot[j] = 0;
            if (j < k && b < B) {
                start[j] = offp[b];
                tot[j] = offp[b + 1] - offp[b];
                if (t < ntiles) base[b] = start[j] + hh[static_cast<size_t>(t) * B + b];
            }
        }
    } else {
        BucketSums bs;
        bucket_sums(O, h, t, ntiles, B, k, bs, pt, pb);
        const int total = bucket_starts(bs, B, k, start, smem);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            tot[j] = bs.total[j];
            if (j < k && b0 + j < B) {
                base[b0 + j] = start[j] + bs.before[j];
                if (lead && offp) offp[b0 + j] = start[j];
            }
        }
        if (lead && offp && tid == 0) offp[B] = total;
    }

    // ---- the attention work list: items in decreasing order of key tiles
    // (ties: lower bucket first), so the longest items start first.  Built by
    // the builder block from both sets' histograms (its ``start`` and
    // ``tot`` above are the query set's; after a scan, both sets' off).
    if (builder) {
        int* qoff = reinterpret_cast<int*>(wcnt[0]);
        int* qcnt = reinterpret_cast<int*>(wcnt[1]);
        int* koff = reinterpret_cast<int*>(wcnt[2]);
        int* kcnt = reinterpret_cast<int*>(wcnt[3]);
        int* slot = run;
        int kstart[4], ktot[4];
        if (a.scanned) {
            const int32_t* ko = KBUF.off + static_cast<size_t>(h) * (B + 1);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int b = b0 + j;
                kstart[j] = ktot[j] = 0;
                if (j < k && b < B) {
                    kstart[j] = ko[b];
                    ktot[j] = ko[b + 1] - ko[b];
                }
            }
        } else {
            int nak;
            const int nkeys = set_count(KSET, h, nak);
            BucketSums ks;
            bucket_sums(KBUF, h, 0, sort_tiles(nkeys), B, k, ks, pt, pb);
            bucket_starts(ks, B, k, kstart, smem);
#pragma unroll
            for (int j = 0; j < 4; ++j) ktot[j] = ks.total[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < k && b0 + j < B) {
                qoff[b0 + j] = start[j];
                qcnt[b0 + j] = tot[j];
                koff[b0 + j] = kstart[j];
                kcnt[b0 + j] = ktot[j];
            }
        }
        __syncthreads();
        const int qt = IT.qtile;
        // rank of bucket b = buckets with more keys, or as many and a lower
        // index; with B <= 256 the 256 / B threads of a bucket split the count
        int rank[4], tiles[4];
        if (k == 1) {
            // B <= 256, bucket b = thread b.  Items are ordered by their key
            // tiles (an item's cost; 255 and more share the top class),
            // larger first, ties by bucket: a stable counting sort of the
            // buckets by class.  Each wave finds the lanes of its own class
            // with one ballot per class bit; per-wave class counts in LDS
            // carry the order across waves.
            int* chist = racc;                       // [256] buckets per class
            int* wcls = base;                        // [4][256] buckets per wave and class
            const int b = tid, w = tid / kWave;
            const bool has = b < B;
            const int cls = has ? min((kcnt[b] + kItemKeyTile - 1) / kItemKeyTile, 255) : 0;
            chist[tid] = 0;
#pragma unroll
            for (int v = 0; v < 4; ++v) wcls[v * 256 + tid] = 0;
            uint64_t same = __ballot(has);
#pragma unroll
            for (int bit = 0; bit < 8; ++bit) {
                const bool on = (cls >> bit) & 1;
                const uint64_t m = __ballot(on);
                same &= on ? m : ~m;
            }
            const int in_wave = __popcll(same & lanemask_lt());
            __syncthreads();
            if (has && in_wave == 0) {               // one lane per (wave, class)
                const int c = __popcll(same);
                wcls[w * 256 + cls] = c;
                atomicAdd(&chist[cls], c);
            }
            __syncthreads();
            // buckets in larger classes: a scan over the classes, largest first
            const int hc = chist[255 - tid];
            int tot_c;
            const int above = block_exclusive_scan<256>(hc, smem, tot_c);
            __syncthreads();
            chist[255 - tid] = above;
            __syncthreads();
            int r = 0;
            if (has) {
                r = chist[cls] + in_wave;
                for (int v = 0; v < w; ++v) r += wcls[v * 256 + cls];
            }
            __syncthreads();
            if (has) racc[b] = r;
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            rank[j] = 0;
            tiles[j] = 0;
            const int b = b0 + j;
            if (j < k && b < B) {
                if (k == 1) {
                    rank[j] = racc[b];
                } else {
                    auto cls_of = [](int kc) { return min((kc + kItemKeyTile - 1) / kItemKeyTile, 255); };
                    const int kn = cls_of(kcnt[b]);
                    for (int c = 0; c < B; ++c) {
                        const int kc = cls_of(kcnt[c]);
                        rank[j] += (kc > kn) || (kc == kn && c < b);
                    }
                }
                tiles[j] = (qcnt[b] + qt - 1) / qt;
                slot[rank[j]] = tiles[j];
            }
        }
        __syncthreads();
        // exclusive prefix of the slice counts in rank order: first item of each rank
        int rs = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) rs += (j < k && b0 + j < B) ? slot[b0 + j] : 0;
        int ntot;
        int first = block_exclusive_scan<256>(rs, smem, ntot);
        int firsts[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            firsts[j] = first;
            first += (j < k && b0 + j < B) ? slot[b0 + j] : 0;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (j < k && b0 + j < B) slot[b0 + j] = firsts[j];     // start of rank b0 + j
        __syncthreads();
        int4* it = IT.items + static_cast<size_t>(h) * IT.max_items;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = b0 + j;
            if (j < k && b < B) {
                const int f0 = slot[rank[j]], qc = qcnt[b];
                for (int c = 0; c < tiles[j]; ++c)
                    it[f0 + c] = make_int4(qoff[b] + c * qt, min(qt, qc - c * qt), koff[b],
                                           kcnt[b]);
            }
        }
        for (int i = ntot + tid; i < IT.max_items; i += 256) it[i] = make_int4(0, 0, 0, 0);
        return;                                   // block uniform
    }
    if (t >= ntiles) return;                      // block uniform

    for (int b = tid; b < B; b += 256) {
        run[b] = 0;
        wcnt[0][b] = wcnt[1][b] = wcnt[2][b] = wcnt[3][b] = 0;
    }
    __syncthreads();
    const int lane = lane_id();
    const int w = threadIdx.x / kWave;
    int32_t* perm = O.perm + static_cast<size_t>(h) * O.perm_stride;
    int rk[R];                                    // the elements' ranks, for the staged write-out
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int e = t * kSortTile + r * 256 + threadIdx.x;
        const bool valid = e < n;
        const int id = idr[r];
        uint64_t mask = __ballot(valid);
        for (int p = 0; p < P; ++p) {
            const bool bit = (id >> p) & 1;
            const uint64_t bb = __ballot(bit);
            mask &= bit ? bb : ~bb;
        }
        const int rank_w = __popcll(mask & lanemask_lt());
        const uint32_t tag = static_cast<uint32_t>(r + 1) << 16;
        if (valid && rank_w == 0) wcnt[w][id] = tag | static_cast<uint32_t>(__popcll(mask));
        __syncthreads();
        int rank = 0;
        bool last = false;
        if (valid) {
            int pre = run[id];
            last = (mask >> lane) == 1;
            for (int v = 0; v < 4; ++v) {
                const uint32_t x = wcnt[v][id];
                const bool cur = (x & 0xFFFF0000u) == tag;
                if (v < w && cur) pre += static_cast<int>(x & 0xFFFFu);
                if (v > w && cur) last = false;
            }
            rank = pre + rank_w;
        }
        __syncthreads();
        rk[r] = rank;
        if (valid) {
            if (last) run[id] = rank + 1;
            if (!a.staged) perm[base[id] + rank] = e;
        }
    }
    if (!a.staged) return;                        // block uniform

    // Staged write-out: run[b] now counts bucket b in this tile.  Its
    // exclusive scan places the tile's elements in bucket order in LDS (each
    // with its global position), and consecutive threads then write
    // consecutive positions of one bucket: runs of stores instead of 4-byte
    // scatter.  wcnt is free again and holds the two arrays.
    __syncthreads();
    {
        const int k = (B + 255) / 256, b0 = tid * k;
        int mine = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) mine += (j < k && b0 + j < B) ? run[b0 + j] : 0;
        int tot;
        int off = block_exclusive_scan<256>(mine, smem, tot);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < k && b0 + j < B) {
                const int c = run[b0 + j];
                run[b0 + j] = off;                // tile-local start of bucket b0 + j
                off += c;
            }
        }
    }
    __syncthreads();
    int* s_pos = reinterpret_cast<int*>(wcnt[0]);
    int* s_e = reinterpret_cast<int*>(wcnt[1]);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int e = t * kSortTile + r * 256 + threadIdx.x;
        if (e < n) {
            const int id = idr[r];
            const int lp = run[id] + rk[r];
            if (lp >= 0 && lp < kSortTile) {      // in range whenever the counts are right
                s_pos[lp] = base[id] + rk[r];
                s_e[lp] = e;
            }
        }
    }
    __syncthreads();
    const int tile_n = min(kSortTile, n - t * kSortTile);
    for (int i = threadIdx.x; i < tile_n; i += 256) perm[s_pos[i]] = s_e[i];
}

hipError_t launch_bucket_sort(int H, int P, int nsets, const IdSet* sets, const SortBufs* bufs,
                              const ItemTable* items, int npairs, hipStream_t s) {
    if (nsets < 1 || nsets > kSortMaxSets || npairs < 0 || npairs > kSortMaxPairs ||
        (npairs > 0 && nsets != 2 * npairs))
        return hipErrorInvalidValue;
    SortArgs a;
    a.nsets = nsets;
    a.npairs = items ? npairs : 0;
    a.builder_block = -1;
    a.B = 1 << P;
    a.P = P;
    for (int i = 0; i < a.npairs; ++i) a.items[i] = items[i];
    int max_tiles = 0;
    for (int i = 0; i < nsets; ++i) {
        a.set[i] = sets[i];
        a.buf[i] = bufs[i];
        if (bufs[i].max_tiles > max_tiles) max_tiles = bufs[i].max_tiles;
    }
    if (H == 0) return hipSuccess;
    // a scan launch once the tiles are many (every set must then have off)
    bool offs = true;
    for (int i = 0; i < nsets; ++i) offs = offs && bufs[i].off != nullptr;
    a.scanned = (max_tiles > kSortScanTiles && offs) ? 1 : 0;
    a.staged = max_tiles >= kSortStagedTiles ? 1 : 0;
    if (max_tiles > 0) {
        timer_begin("sort_hist", s);
        hipLaunchKernelGGL(sort_hist_kernel, dim3(max_tiles, H, nsets), dim3(256), 0, s, a);
        timer_end(s);
    }
    if (a.scanned) {
        timer_begin("sort_scan", s);
        hipLaunchKernelGGL(sort_scan_kernel, dim3(H, nsets), dim3(kScanNT), 0, s, a);
        timer_end(s);
    }
    int gx = max_tiles > 0 ? max_tiles : 1;
    if (a.npairs > 0) a.builder_block = gx++;
    timer_begin("sort_scatter", s);
    hipLaunchKernelGGL(sort_scatter_kernel, dim3(gx, H, nsets), dim3(256), 0, s, a);
    timer_end(s);
    return hipGetLastError();
}

}  // namespace fastar
