// Stable counting sort of token indices by bucket id: the block-sparse layout
// that bucket attention gathers from (FAST-AR summary, "2. Core Components",
// part C).  Three launches, every count stays on the device:
//
//   sort_hist    one block per 1024-id tile: LDS histogram -> hist[h][tile][b]
//   sort_scan    one block per head: per-bucket exclusive prefix over tiles (in
//                place) plus a block scan over buckets -> off[h][b], for each
//                set; optionally the attention work list (one item per bucket
//                and 64-query slice, longest key lists first)
//   sort_scatter one block per tile: stable rank of every id inside its tile
//                (wave ballots on the P id bits give the rank among equal ids of
//                the wave; LDS counters tagged by round carry it across waves
//                and rounds), then perm[off + tile base + rank] = index.
//
// The result is unique (a stable sort), so it is bit-identical run to run.
#include "common.hpp"
#include "launch.hpp"

namespace fastar {

struct SortArgs {
    IdSet set[2];
    SortBufs buf[2];
    int nsets;
    int B;
    int P;
    ItemTable items;
};

__device__ __forceinline__ int set_count(const IdSet& s, int h, int& na) {
    na = s.a_nvalid ? clamp_n(s.a_nvalid, h, s.a_cap) : s.a_fixed;
    return na + s.nb;
}

__device__ __forceinline__ int set_id(const IdSet& s, int h, int na, int e) {
    return e < na ? s.a[static_cast<size_t>(h) * s.a_stride + e]
                  : s.b[static_cast<size_t>(h) * s.b_stride + (e - na)];
}

__global__ __launch_bounds__(256) void sort_hist_kernel(SortArgs a) {
    __shared__ int cnt[1024];
    const IdSet& S = a.set[blockIdx.z];
    const SortBufs& O = a.buf[blockIdx.z];
    const int h = blockIdx.y, t = blockIdx.x, B = a.B;
    int na;
    const int n = set_count(S, h, na);
    if (t * kSortTile >= n) return;
    for (int b = threadIdx.x; b < B; b += 256) cnt[b] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSortTile / 256; ++r) {
        const int e = t * kSortTile + r * 256 + threadIdx.x;
        if (e < n) atomicAdd(&cnt[(set_id(S, h, na, e) >> S.shift) & (B - 1)], 1);
    }
    __syncthreads();
    int* dst = O.hist + (static_cast<size_t>(h) * O.max_tiles + t) * B;
    for (int b = threadIdx.x; b < B; b += 256) dst[b] = cnt[b];
}

// One block per head.  Thread (part, b) owns bucket b over a contiguous range
// of tiles (1024 / B parts), so every tile count is read by one thread.  When
// a part spans at most kScanRegs tiles (the usual case) the counts of both sets
// are loaded into registers up front -- one round trip for the whole kernel --
// and the running offsets are written back from them; longer parts loop.
constexpr int kScanRegs = 8;

__global__ __launch_bounds__(1024) void sort_scan_kernel(SortArgs a) {
    __shared__ int part_sum[1024];
    __shared__ int smem[16];
    __shared__ int offs[2][1025];
    __shared__ int rank_acc[1024];
    const int h = blockIdx.x, B = a.B, tid = threadIdx.x;
    const int parts = 1024 / B;
    const int b = tid % B, part = tid / B;
    rank_acc[tid] = 0;                    // ordered before its use by the scans' barriers
    int cnt[2][kScanRegs];
    int t0s[2], t1s[2];
    bool regs[2];
#pragma unroll
    for (int si = 0; si < 2; ++si) {
        t0s[si] = t1s[si] = 0;
        regs[si] = true;
        if (si >= a.nsets) continue;
        int na;
        const int n = set_count(a.set[si], h, na);
        const int ntiles = sort_tiles(n);
        const int tpp = (ntiles + parts - 1) / parts;
        t0s[si] = min(ntiles, part * tpp);
        t1s[si] = min(ntiles, t0s[si] + tpp);
        regs[si] = tpp <= kScanRegs;                               // block uniform
        const int* hist = a.buf[si].hist + static_cast<size_t>(h) * a.buf[si].max_tiles * B + b;
#pragma unroll
        for (int k = 0; k < kScanRegs; ++k)
            cnt[si][k] = (regs[si] && t0s[si] + k < t1s[si]) ? hist[static_cast<size_t>(t0s[si] + k) * B] : 0;
    }
#pragma unroll
    for (int si = 0; si < 2; ++si) {
        if (si >= a.nsets) break;
        const SortBufs& O = a.buf[si];
        const int t0 = t0s[si], t1 = t1s[si];
        int* hist = O.hist + static_cast<size_t>(h) * O.max_tiles * B + b;
        int sum = 0;
        if (regs[si]) {
#pragma unroll
            for (int k = 0; k < kScanRegs; ++k) sum += cnt[si][k];
        } else {
#pragma unroll 4
            for (int t = t0; t < t1; ++t) sum += hist[static_cast<size_t>(t) * B];
        }
        part_sum[part * B + b] = sum;
        __syncthreads();
        int pre = 0, tot = 0;
        for (int q = 0; q < parts; ++q) {
            const int v = part_sum[q * B + b];
            pre += (q < part) ? v : 0;
            tot += v;
        }
        int total;
        const int excl = block_exclusive_scan<1024>(part == 0 ? tot : 0, smem, total);
        if (part == 0) offs[si][b] = excl;
        if (tid == 0) offs[si][B] = total;
        __syncthreads();
        int run = offs[si][b] + pre;
        if (regs[si]) {
#pragma unroll
            for (int k = 0; k < kScanRegs; ++k) {
                if (t0 + k < t1) hist[static_cast<size_t>(t0 + k) * B] = run;
                run += cnt[si][k];
            }
        } else {
            for (int t = t0; t < t1; ++t) {
                const int c = hist[static_cast<size_t>(t) * B];
                hist[static_cast<size_t>(t) * B] = run;
                run += c;
            }
        }
        if (part == 0) O.off[static_cast<size_t>(h) * (B + 1) + b] = offs[si][b];
        if (tid == 0) O.off[static_cast<size_t>(h) * (B + 1) + B] = total;
    }
    if (a.items.items && a.nsets == 2) {
        // Items in decreasing order of key count (ties: lower bucket first), so
        // the longest items start first.  rank[b] = position of bucket b.
        // every part counts the buckets of its share of c that rank before b
        __shared__ int slot_tiles[1024];
        const int qc = (part == 0) ? offs[0][b + 1] - offs[0][b] : 0;
        const int kn = offs[1][b + 1] - offs[1][b];
        const int tiles = (qc + kQTile - 1) / kQTile;
        const int per = (B + parts - 1) / parts;
        int r = 0;
        for (int c = part * per; c < min(B, (part + 1) * per); ++c) {
            const int kc = offs[1][c + 1] - offs[1][c];
            r += (kc > kn) || (kc == kn && c < b);
        }
        atomicAdd(&rank_acc[b], r);
        __syncthreads();
        const int rank = rank_acc[b];
        if (part == 0) slot_tiles[rank] = tiles;
        __syncthreads();
        int ntot;
        const int first_by_rank = block_exclusive_scan<1024>(part == 0 ? slot_tiles[b] : 0, smem, ntot);
        if (part == 0) slot_tiles[b] = first_by_rank;          // start of rank b
        __syncthreads();
        int4* it = a.items.items + static_cast<size_t>(h) * a.items.max_items;
        if (part == 0) {
            const int first = slot_tiles[rank];
            const int ks = offs[1][b];
            for (int c = 0; c < tiles; ++c)
                it[first + c] = make_int4(offs[0][b] + c * kQTile, min(kQTile, qc - c * kQTile), ks, kn);
        }
        for (int i = ntot + tid; i < a.items.max_items; i += 1024) it[i] = make_int4(0, 0, 0, 0);
    }
}

__global__ __launch_bounds__(256) void sort_scatter_kernel(SortArgs a) {
    __shared__ int run[1024];
    __shared__ int base[1024];
    __shared__ uint32_t wcnt[4][1024];
    const IdSet& S = a.set[blockIdx.z];
    const SortBufs& O = a.buf[blockIdx.z];
    const int h = blockIdx.y, t = blockIdx.x, B = a.B, P = a.P;
    int na;
    const int n = set_count(S, h, na);
    if (t * kSortTile >= n) return;
    const int* tb = O.hist + (static_cast<size_t>(h) * O.max_tiles + t) * B;
    for (int b = threadIdx.x; b < B; b += 256) {
        run[b] = 0;
        base[b] = tb[b];
        wcnt[0][b] = wcnt[1][b] = wcnt[2][b] = wcnt[3][b] = 0;
    }
    __syncthreads();
    const int lane = lane_id();
    const int w = threadIdx.x / kWave;
    int32_t* perm = O.perm + static_cast<size_t>(h) * O.perm_stride;
#pragma unroll 1
    for (int r = 0; r < kSortTile / 256; ++r) {
        const int e = t * kSortTile + r * 256 + threadIdx.x;
        const bool valid = e < n;
        const int id = valid ? ((set_id(S, h, na, e) >> S.shift) & (B - 1)) : 0;
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
        if (valid) {
            if (last) run[id] = rank + 1;
            perm[base[id] + rank] = e;
        }
    }
}

hipError_t launch_bucket_sort(int H, int P, int nsets, const IdSet* sets, const SortBufs* bufs,
                              const ItemTable* items, hipStream_t s) {
    SortArgs a;
    a.nsets = nsets;
    a.B = 1 << P;
    a.P = P;
    a.items = items ? *items : ItemTable();
    int max_tiles = 0;
    for (int i = 0; i < nsets; ++i) {
        a.set[i] = sets[i];
        a.buf[i] = bufs[i];
        if (bufs[i].max_tiles > max_tiles) max_tiles = bufs[i].max_tiles;
    }
    if (nsets == 1) {
        a.set[1] = a.set[0];
        a.buf[1] = a.buf[0];
    }
    if (H == 0) return hipSuccess;
    if (max_tiles > 0) {
        timer_begin("sort_hist", s);
        hipLaunchKernelGGL(sort_hist_kernel, dim3(max_tiles, H, nsets), dim3(256), 0, s, a);
        timer_end(s);
    }
    timer_begin("sort_scan", s);
    hipLaunchKernelGGL(sort_scan_kernel, dim3(H), dim3(1024), 0, s, a);
    timer_end(s);
    if (max_tiles > 0) {
        timer_begin("sort_scatter", s);
        hipLaunchKernelGGL(sort_scatter_kernel, dim3(max_tiles, H, nsets), dim3(256), 0, s, a);
        timer_end(s);
    }
    return hipGetLastError();
}

}  // namespace fastar
