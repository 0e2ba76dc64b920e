// Host-side launchers of the FAST-AR kernels (defined in the .hip files),
// called by the C ABI after it has validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fastar {

// Per-kernel timing hooks (capi.cpp); no-ops unless fastar_timer_start is active.
void timer_begin(const char* name, hipStream_t s);
void timer_end(hipStream_t s);

// ------------------------------------------------------------------ hash
constexpr int kHashBatch = 4;          // token sets per batched launch
hipError_t launch_hash(const void* x, bool bf16, int H, int N, int d, const float* planes, int P,
                       uint16_t* ids, float* norms, hipStream_t s);
// ``count`` <= kHashBatch sets (host arrays); ``norms`` may be null, or hold
// null entries.
hipError_t launch_hash_batch(int count, const void* const* x, const int* N, uint16_t* const* ids,
                             float* const* norms, bool bf16, int H, int d, const float* planes, int P,
                             hipStream_t s);

// ------------------------------------------------------------------ quantization ids
hipError_t launch_quantize(const void* x, bool bf16, int H, int N, int d, const float* codebook, int B,
                           uint16_t* ids, float* norms, hipStream_t s);
// ``count`` <= kHashBatch sets (host arrays), as launch_hash_batch.
hipError_t launch_quantize_batch(int count, const void* const* x, const int* N, uint16_t* const* ids,
                                 float* const* norms, bool bf16, int H, int d, const float* codebook, int B,
                                 hipStream_t s);

// ------------------------------------------------------------------ sort
// A set of ids per head: the first part (source a) holds either ``a_fixed``
// ids or, when ``a_nvalid`` is set, clamp(a_nvalid[h], 0, a_cap) ids; the
// second part (source b) holds ``nb`` ids.  Element e of the set is a[e] for
// e < na, b[e - na] otherwise.
struct IdSet {
    int shift = 0;             // bucket id = (id >> shift) & (2^P - 1): table field of a multi-table id
    const uint16_t* a = nullptr;
    int a_stride = 0;          // ids per head in a's array
    int a_fixed = 0;
    const int32_t* a_nvalid = nullptr;
    int a_cap = 0;
    const uint16_t* b = nullptr;
    int b_stride = 0;
    int nb = 0;
};

struct SortBufs {
    int32_t* hist = nullptr;    // [H][max_tiles][B] scratch (tile counts, then tile bases)
    int32_t* off = nullptr;     // [H][B+1]
    int32_t* perm = nullptr;    // [H][perm_stride]
    int max_tiles = 0;
    int perm_stride = 0;
};

constexpr int kSortTile = 1024;
constexpr int kQTile = 64;   // queries per attention block
// queries per block of the wide AnnSA kernel (8 waves x 2 groups of 16),
// used when buckets average at least this many queries
constexpr int kQTileWide = 256;
__host__ __device__ inline int sort_tiles(long long n) { return static_cast<int>((n + kSortTile - 1) / kSortTile); }

// Attention work items built from a (query set, key set) pair of groupings:
// one item per (bucket, qtile-query slice) with at least one query, in bucket
// order: x = first query position in the query permutation, y = number of
// queries (0 marks padding), z = first key position, w = number of keys.
struct ItemTable {
    int4* items = nullptr;      // [H][max_items]
    int max_items = 0;
    int qtile = kQTile;         // queries per item: kQTile or kQTileWide
};
// Upper bound on the number of items of one head (a multiple of 8).
inline int max_attn_items(long long nq, int B) {
    long long m = (nq + kQTile - 1) / kQTile + B;
    return static_cast<int>((m + 7) / 8 * 8);
}

// Sorts ``nsets`` sets per head (at most kSortMaxSets): a tile-histogram
// launch and a scatter launch (plus a scan launch between them when a set
// spans more than kSortScanTiles tiles).  With ``items`` (an array of
// ``npairs`` tables; the sets then form npairs (queries, keys) pairs) one
// more scatter block per head and pair writes that pair's attention work list.
constexpr int kSortMaxPairs = 8;            // FASTAR_MAX_TABLES
constexpr int kSortMaxSets = 2 * kSortMaxPairs;
hipError_t launch_bucket_sort(int H, int P, int nsets, const IdSet* sets, const SortBufs* bufs,
                              const ItemTable* items, int npairs, hipStream_t s);

// ------------------------------------------------------------------ attention
enum AttnMode { MODE_SA = 0, MODE_CA = 1, MODE_TOP1 = 2 };

struct AttnParams {
    int H = 0;                      // heads (set by launch_attn)
    const void* q = nullptr;        // [H][Nq][D]
    int Nq = 0;
    // key/value rows: source a (cache slots, or prompt rows), source b (current chunk)
    const void* ka = nullptr;
    const void* va = nullptr;
    int a_rows = 0;                 // rows per head in source a
    const void* kb = nullptr;
    const void* vb = nullptr;
    int b_rows = 0;
    const int32_t* n_valid = nullptr;
    int cap = 0;
    const float* knorm = nullptr;   // [H][a_rows] key norms of source a (search)
    const int32_t* kcount = nullptr; // [H][a_rows] group sizes of source a (mean-merged cache)
    // multi-table AnnSA (tables > 1): one launch per table; ids hold a P-bit
    // field per table; pairs already matched by an earlier table are masked,
    // and the online-softmax / search state carries over between launches
    int table = 0, tables = 1, fbits = 0;
    int wide = 0;               // AnnSA items of kQTileWide queries (the wide kernel)
    const uint16_t* q_ids = nullptr;  // [H][Nq]
    const uint16_t* ida = nullptr;    // [H][a_rows] ids of source a
    const uint16_t* idb = nullptr;    // [H][b_rows] ids of source b
    float* st_o = nullptr;            // [H][Nq][D] unnormalised output
    float* st_m = nullptr;            // [H][Nq] softmax reference maximum (raw score units)
    float* st_l = nullptr;            // [H][Nq] running sum
    float* st_bc = nullptr;           // [H][Nq] search: best dot/|k|
    int32_t* st_bs = nullptr;         // [H][Nq] search: its slot
    // bucket groupings and work items (SA, TOP1)
    const int32_t* qperm = nullptr;
    int qperm_stride = 0;
    const int32_t* kperm = nullptr;
    int kperm_stride = 0;
    const int4* items = nullptr;
    int max_items = 0;              // work-list entries per head (a multiple of 8)
    // prompt selection (CA)
    const int32_t* ca_idx = nullptr;
    const int32_t* ca_cnt = nullptr;
    int frame_len = 0;
    int F = 0;
    int L = 0;
    // prompt selection fused into the AnnCA blocks (ca_fused = 1, L <=
    // kCaFusedMaxL): the prompt's bucket ids (null when L = 0), the bucket
    // count and the keep outputs (either may be null); with ca_fused = 0 the
    // blocks read ca_idx / ca_cnt instead
    int ca_fused = 0;
    const uint16_t* ca_kp_ids = nullptr;
    int ca_buckets = 0;
    uint8_t* ca_keep = nullptr;
    int32_t* ca_keep_count = nullptr;
    // outputs
    void* out = nullptr;
    float* lse = nullptr;
    int32_t* best = nullptr;
    float* bcos = nullptr;
    float scale_log2 = 0.f;
};

// Longest prompt whose kept list an AnnCA block builds in its own LDS, and
// the most buckets its bitmap holds (2^10, the bucketed calls' plane limit).
constexpr int kCaFusedMaxL = 1024;
constexpr int kCaMaxBuckets = 1024;

hipError_t launch_attn(int mode, bool bf16, int d, bool out_bf16, int H, const AttnParams& p,
                       hipStream_t s);

// ------------------------------------------------------------------ AnnCA selection
hipError_t launch_annca_select(const uint16_t* q_ids, const uint16_t* kp_ids, int H, int Nq,
                               int frame_len, int L, int P, int32_t* idx, int32_t* cnt,
                               uint8_t* keep, int32_t* keep_count, hipStream_t s);

// ------------------------------------------------------------------ TempCache commit
struct TcSelectParams {
    const int32_t* best;     // [H][N]
    const float* cosv;       // [H][N]
    int32_t* claim;          // [H][cap] scratch; only the entries of matched slots are used
    uint32_t* refreshed;     // [H][ceil(cap/32)] scratch bitmap
    const int32_t* ts;       // [H][cap]
    int32_t* n_valid;        // [H] read, then updated
    int32_t* upos;           // [H][N] scratch
    int32_t* ev;             // [H][N] scratch: evicted slots, ascending
    int32_t* dest;           // [H][N] output (scratch or caller's)
    int32_t* evicted;        // [H][N] caller output or null
    int32_t* counts;         // [H][5] caller output or null
    const int32_t* order;    // [H][N] eviction candidates (launch_tc_order) or null
    // mean merge only (null otherwise): the matched tokens grouped by the
    // token that represents their slot
    int32_t* grp_cnt;        // [H][N] scratch: group size of each representative, else 0
    int32_t* grp_off;        // [H][N] scratch: exclusive scan of grp_cnt
    int32_t* grp_mem;        // [H][N] scratch: members of each group (unordered)
    int32_t* grp_pos;        // [H][N] scratch: a member's position in its group
    int H, N, cap;
    float tau;
};
hipError_t launch_tc_select(const TcSelectParams& p, hipStream_t s);
// The min(n_valid, N) slots of smallest (ts, slot) per head, ascending, -1
// padded to N: the candidates of the next commit's eviction search.
hipError_t launch_tc_order(const int32_t* ts, const int32_t* n_valid, int H, int cap, int N, int32_t* order,
                           hipStream_t s);

hipError_t launch_tc_scatter(bool bf16, int d, int H, int N, int cap, const int32_t* dest,
                             const void* k_cur, const void* v_cur, const uint16_t* kcur_ids,
                             int32_t step, void* ck, void* cv, uint16_t* cids, int32_t* cts,
                             float* cnorm, hipStream_t s);
// Mean-merge variant of the scatter: representatives fold their group's
// values into the slot (grp_* as written by the select), the other written
// tokens start groups of one.
hipError_t launch_tc_merge_scatter(bool bf16, int d, int H, int N, int cap, const int32_t* dest,
                                   const int32_t* grp_cnt, const int32_t* grp_off,
                                   const int32_t* grp_mem, const void* k_cur, const void* v_cur,
                                   const uint16_t* kcur_ids, int32_t step, void* ck, void* cv,
                                   uint16_t* cids, int32_t* cts, float* cnorm, int32_t* ccount,
                                   hipStream_t s);

}  // namespace fastar
