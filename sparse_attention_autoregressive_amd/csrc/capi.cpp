// C ABI of the FAST-AR attention step: argument validation, workspace layout
// and kernel sequencing.  Nothing here allocates device memory or waits on the
// device (except fastar_timer_stop, which waits for its own events).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "fastar.h"
#include "annsa_entry.hpp"
#include "launch.hpp"

namespace fastar {

// ------------------------------------------------------------------ timer
// The measurement timer's state is per host thread: a thread's
// fastar_timer_start / fastar_timer_stop see only the launches that thread
// enqueued, and threads never share it.  Every other call keeps no state.
namespace {
struct TimerRec {
    const char* name;
    hipEvent_t a, b;
};
thread_local bool g_timer_on = false;
thread_local bool g_pending = false;
thread_local std::vector<TimerRec> g_recs;
thread_local std::vector<hipEvent_t> g_pool;
thread_local size_t g_pool_used = 0;

hipEvent_t pool_get() {
    if (g_pool_used < g_pool.size()) return g_pool[g_pool_used++];
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_pool.push_back(e);
    ++g_pool_used;
    return e;
}
}  // namespace

void timer_begin(const char* name, hipStream_t s) {
    g_pending = false;
    if (!g_timer_on || g_recs.size() >= FASTAR_TIMER_MAX) return;
    // a stream being captured into a graph gets no event nodes
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return;
    hipEvent_t a = pool_get(), b = pool_get();
    if (!a || !b || hipEventRecord(a, s) != hipSuccess) return;
    g_recs.push_back({name, a, b});
    g_pending = true;
}

void timer_end(hipStream_t s) {
    if (!g_pending) return;
    (void)hipEventRecord(g_recs.back().b, s);
    g_pending = false;
}

}  // namespace fastar

using namespace fastar;

namespace {

// Workspace carving: the size queries and the calls run the same plan, one with
// a null base (sizing), one with the caller's pointer.
struct Carver {
    char* base;
    size_t off = 0;
    explicit Carver(void* b) : base(static_cast<char*>(b)) {}
    template <typename T>
    T* take(long long count) {
        const size_t bytes = static_cast<size_t>(count > 0 ? count : 0) * sizeof(T);
        T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
        off += (bytes + 255) & ~static_cast<size_t>(255);
        return p;
    }
};

SortBufs carve_sort(Carver& c, int H, long long nmax, int P, bool with_off_perm) {
    SortBufs s;
    const int B = 1 << P;
    s.max_tiles = sort_tiles(nmax);
    s.perm_stride = static_cast<int>(nmax);
    s.hist = c.take<int32_t>(static_cast<long long>(H) * s.max_tiles * B);
    if (with_off_perm) {
        s.off = c.take<int32_t>(static_cast<long long>(H) * (B + 1));
        s.perm = c.take<int32_t>(static_cast<long long>(H) * nmax);
    }
    return s;
}

ItemTable carve_items(Carver& c, int H, long long nq, int P) {
    ItemTable t;
    t.max_items = max_attn_items(nq, 1 << P);
    t.items = c.take<int4>(static_cast<long long>(H) * t.max_items);
    return t;
}

// One (queries, keys) sort and work list per hash table: multi-table calls
// sort every table's fields in one launch pair.
struct AnnsaWs {
    SortBufs q[FASTAR_MAX_TABLES], k[FASTAR_MAX_TABLES];
    ItemTable it[FASTAR_MAX_TABLES];
};
AnnsaWs carve_annsa(Carver& c, int H, int Nq, int cap, int Ncur, int P, int tables = 1) {
    AnnsaWs w;
    for (int t = 0; t < tables; ++t) {
        w.q[t] = carve_sort(c, H, Nq, P, true);
        w.k[t] = carve_sort(c, H, static_cast<long long>(cap) + Ncur, P, true);
        w.it[t] = carve_items(c, H, Nq, P);
    }
    return w;
}

// Multi-table AnnSA: each query's online-softmax and search state between
// the per-table launches.
struct StateWs {
    float *o = nullptr, *m = nullptr, *l = nullptr, *bc = nullptr;
    int32_t* bs = nullptr;
};
StateWs carve_state(Carver& c, int H, int Nq, int d, int tables) {
    StateWs w;
    if (tables <= 1) return w;
    const long long HQ = static_cast<long long>(H) * Nq;
    w.o = c.take<float>(HQ * d);
    w.m = c.take<float>(HQ);
    w.l = c.take<float>(HQ);
    w.bc = c.take<float>(HQ);
    w.bs = c.take<int32_t>(HQ);
    return w;
}

struct AnncaWs {
    int32_t* idx;
    int32_t* cnt;
};
AnncaWs carve_annca(Carver& c, int H, int F, int L) {
    AnncaWs w;
    w.idx = c.take<int32_t>(static_cast<long long>(H) * F * L);
    w.cnt = c.take<int32_t>(static_cast<long long>(H) * F);
    return w;
}

struct TcWs {
    SortBufs q, k;
    ItemTable it;
    int32_t *claim, *best, *upos, *ev, *dest;
    int32_t *grp_cnt, *grp_off, *grp_mem, *grp_pos;   // mean merge
    uint32_t* refreshed;
    float* cosv;
};
TcWs carve_tc(Carver& c, int H, int N, int cap, int P) {
    TcWs w;
    w.q = carve_sort(c, H, N, P, true);
    w.k = carve_sort(c, H, cap, P, true);
    w.it = carve_items(c, H, N, P);
    const long long HN = static_cast<long long>(H) * N;
    w.claim = c.take<int32_t>(static_cast<long long>(H) * cap);
    w.refreshed = c.take<uint32_t>(static_cast<long long>(H) * ((cap + 31) / 32));
    w.best = c.take<int32_t>(HN);
    w.cosv = c.take<float>(HN);
    w.upos = c.take<int32_t>(HN);
    w.ev = c.take<int32_t>(HN);
    w.dest = c.take<int32_t>(HN);
    w.grp_cnt = c.take<int32_t>(HN);
    w.grp_off = c.take<int32_t>(HN);
    w.grp_mem = c.take<int32_t>(HN);
    w.grp_pos = c.take<int32_t>(HN);
    return w;
}

bool dtype_ok(int dt) { return dt == FASTAR_F32 || dt == FASTAR_BF16; }
bool d_ok(int d) { return d == 64 || d == 128; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool planes_ok(int P) { return P >= 0 && P <= FASTAR_MAX_PLANES; }
// Tables of P bits each share one 16-bit id.
bool tables_ok(int P, int tables) {
    return tables >= 1 && tables <= FASTAR_MAX_TABLES && P * tables <= FASTAR_MAX_HASH_PLANES;
}

// Tensor pointer rule: required when the tensor is non-empty, 16-byte aligned when given.
bool tensor_ok(const void* p, long long elems) {
    if (elems <= 0) return p == nullptr || aligned16(p);
    return p != nullptr && aligned16(p);
}
bool small_ok(const void* p, long long elems) { return elems <= 0 || p != nullptr; }
bool fits_i32(long long v) { return v >= 0 && v < (1ll << 31); }
// One head's rows of a K/V tensor are addressed with 32-bit byte offsets.
bool head_bytes_ok(long long rows, int d, int dtype) {
    return rows * d * (dtype == FASTAR_BF16 ? 2 : 4) < (1ll << 32);
}

fastar_status hip_status(hipError_t e) { return e == hipSuccess ? FASTAR_OK : FASTAR_EHIP; }

bool cache_ok(const fastar_cache* c, int H, int d, int dtype) {
    if (!c) return true;
    if (c->H != H || c->d != d || c->dtype != dtype || c->cap < 0) return false;
    const long long rows = static_cast<long long>(H) * c->cap;
    if (!fits_i32(rows * d)) return false;
    return tensor_ok(c->k, rows * d) && tensor_ok(c->v, rows * d) && small_ok(c->ids, rows) &&
           small_ok(c->ts, rows) && small_ok(c->knorm, rows) && small_ok(c->n_valid, H);
}

}  // namespace

extern "C" {

const char* fastar_status_string(int32_t status) {
    switch (status) {
        case FASTAR_OK: return "FASTAR_OK";
        case FASTAR_EINVAL: return "FASTAR_EINVAL";
        case FASTAR_EDTYPE: return "FASTAR_EDTYPE";
        case FASTAR_ESHAPE: return "FASTAR_ESHAPE";
        case FASTAR_EWORKSPACE: return "FASTAR_EWORKSPACE";
        case FASTAR_ECAPACITY: return "FASTAR_ECAPACITY";
        case FASTAR_EHIP: return "FASTAR_EHIP";
        case FASTAR_ESCRATCH: return "FASTAR_ESCRATCH";
        default: return "FASTAR_UNKNOWN";
    }
}

int32_t fastar_abi_version(void) { return FASTAR_ABI_VERSION; }

// ------------------------------------------------------------------ hash
fastar_status fastar_ann_hash(const void* x, int32_t dtype, int32_t H, int32_t N, int32_t d,
                              const float* planes, int32_t P, uint16_t* ids, float* norms,
                              void* stream) {
    if (!dtype_ok(dtype)) return FASTAR_EDTYPE;
    if (H < 0 || N < 0) return FASTAR_EINVAL;
    if (!d_ok(d) || P < 0 || P > FASTAR_MAX_HASH_PLANES) return FASTAR_ESHAPE;
    const long long HN = static_cast<long long>(H) * N;
    if (!fits_i32(HN * d)) return FASTAR_EINVAL;
    if (!tensor_ok(x, HN * d) || !small_ok(ids, HN)) return FASTAR_EINVAL;
    if (!tensor_ok(planes, (HN > 0 ? static_cast<long long>(H) * P * d : 0))) return FASTAR_EINVAL;
    if (HN == 0) return FASTAR_OK;
    return hip_status(launch_hash(x, dtype == FASTAR_BF16, H, N, d, planes, P, ids, norms,
                                  static_cast<hipStream_t>(stream)));
}

fastar_status fastar_ann_hash_batch(int32_t count, const void* const* x, const int32_t* N,
                                    uint16_t* const* ids, float* const* norms, int32_t dtype,
                                    int32_t H, int32_t d, const float* planes, int32_t P,
                                    void* stream) {
    static_assert(FASTAR_HASH_BATCH == kHashBatch, "batch size");
    if (!dtype_ok(dtype)) return FASTAR_EDTYPE;
    if (count < 1 || count > FASTAR_HASH_BATCH || !x || !N || !ids || H < 0) return FASTAR_EINVAL;
    if (!d_ok(d) || P < 0 || P > FASTAR_MAX_HASH_PLANES) return FASTAR_ESHAPE;
    int n[FASTAR_HASH_BATCH];
    long long total = 0;
    for (int i = 0; i < count; ++i) {
        if (N[i] < 0) return FASTAR_EINVAL;
        const long long HN = static_cast<long long>(H) * N[i];
        if (!fits_i32(HN * d)) return FASTAR_EINVAL;
        if (!tensor_ok(x[i], HN * d) || !small_ok(ids[i], HN)) return FASTAR_EINVAL;
        n[i] = N[i];
        total += HN;
    }
    if (!tensor_ok(planes, total > 0 ? static_cast<long long>(H) * P * d : 0)) return FASTAR_EINVAL;
    if (total == 0) return FASTAR_OK;
    return hip_status(launch_hash_batch(count, x, n, ids, norms, dtype == FASTAR_BF16, H, d, planes, P,
                                        static_cast<hipStream_t>(stream)));
}

fastar_status fastar_ann_quantize(const void* x, int32_t dtype, int32_t H, int32_t N, int32_t d,
                                  const float* codebook, int32_t B, uint16_t* ids, float* norms,
                                  void* stream) {
    if (!dtype_ok(dtype)) return FASTAR_EDTYPE;
    if (H < 0 || N < 0) return FASTAR_EINVAL;
    if (!d_ok(d) || B < 1 || B > FASTAR_MAX_CODEWORDS) return FASTAR_ESHAPE;
    const long long HN = static_cast<long long>(H) * N;
    if (!fits_i32(HN * d) || !fits_i32(static_cast<long long>(H) * B * d)) return FASTAR_EINVAL;
    if (!tensor_ok(x, HN * d) || !small_ok(ids, HN)) return FASTAR_EINVAL;
    if (!tensor_ok(codebook, (HN > 0 ? static_cast<long long>(H) * B * d : 0))) return FASTAR_EINVAL;
    if (HN == 0) return FASTAR_OK;
    return hip_status(launch_quantize(x, dtype == FASTAR_BF16, H, N, d, codebook, B, ids, norms,
                                      static_cast<hipStream_t>(stream)));
}

fastar_status fastar_ann_quantize_batch(int32_t count, const void* const* x, const int32_t* N,
                                        uint16_t* const* ids, float* const* norms, int32_t dtype,
                                        int32_t H, int32_t d, const float* codebook, int32_t B,
                                        void* stream) {
    if (!dtype_ok(dtype)) return FASTAR_EDTYPE;
    if (count < 1 || count > FASTAR_HASH_BATCH || !x || !N || !ids || H < 0) return FASTAR_EINVAL;
    if (!d_ok(d) || B < 1 || B > FASTAR_MAX_CODEWORDS) return FASTAR_ESHAPE;
    if (!fits_i32(static_cast<long long>(H) * B * d)) return FASTAR_EINVAL;
    int n[FASTAR_HASH_BATCH];
    long long total = 0;
    for (int i = 0; i < count; ++i) {
        if (N[i] < 0) return FASTAR_EINVAL;
        const long long HN = static_cast<long long>(H) * N[i];
        if (!fits_i32(HN * d)) return FASTAR_EINVAL;
        if (!tensor_ok(x[i], HN * d) || !small_ok(ids[i], HN)) return FASTAR_EINVAL;
        n[i] = N[i];
        total += HN;
    }
    if (!tensor_ok(codebook, total > 0 ? static_cast<long long>(H) * B * d : 0)) return FASTAR_EINVAL;
    if (total == 0) return FASTAR_OK;
    return hip_status(launch_quantize_batch(count, x, n, ids, norms, dtype == FASTAR_BF16, H, d, codebook, B,
                                            static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ bucket sort
size_t fastar_bucket_sort_workspace(int32_t H, int32_t N, int32_t P) {
    if (H < 0 || N < 0 || !planes_ok(P)) return 0;
    Carver c(nullptr);
    carve_sort(c, H, N, P, false);
    return c.off;
}

fastar_status fastar_bucket_sort(const uint16_t* ids, int32_t H, int32_t N, int32_t P,
                                 int32_t* off, int32_t* perm, void* ws, size_t ws_bytes,
                                 void* stream) {
    if (H < 0 || N < 0) return FASTAR_EINVAL;
    if (!planes_ok(P)) return FASTAR_ESHAPE;
    const long long HN = static_cast<long long>(H) * N;
    if (!fits_i32(HN)) return FASTAR_EINVAL;
    if (!small_ok(ids, HN) || !small_ok(perm, HN) || !small_ok(off, H)) return FASTAR_EINVAL;
    const size_t need = fastar_bucket_sort_workspace(H, N, P);
    if (ws_bytes < need || (need > 0 && !ws)) return FASTAR_EWORKSPACE;
    if (H == 0) return FASTAR_OK;
    Carver c(ws);
    SortBufs b = carve_sort(c, H, N, P, false);
    b.off = off;
    b.perm = perm;
    IdSet s;
    s.a = ids;
    s.a_stride = N;
    s.a_fixed = N;
    return hip_status(launch_bucket_sort(H, P, 1, &s, &b, nullptr, 0, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------------ AnnSA
size_t fastar_annsa_workspace(int32_t H, int32_t Nq, int32_t cap, int32_t Ncur, int32_t P) {
    if (H < 0 || Nq < 0 || cap < 0 || Ncur < 0 || !planes_ok(P)) return 0;
    Carver c(nullptr);
    carve_annsa(c, H, Nq, cap, Ncur, P);
    return c.off;
}

size_t fastar_annsa_multi_workspace(int32_t H, int32_t Nq, int32_t cap, int32_t Ncur, int32_t d,
                                    int32_t P, int32_t tables) {
    if (H < 0 || Nq < 0 || cap < 0 || Ncur < 0 || !d_ok(d) || !tables_ok(P, tables)) return 0;
    Carver c(nullptr);
    carve_annsa(c, H, Nq, cap, Ncur, P, tables);
    carve_state(c, H, Nq, d, tables);
    return c.off;
}

}  // extern "C"

namespace fastar {

fastar_status annsa_validate(const void* q, const uint16_t* q_ids, int32_t H, int32_t Nq, int32_t d,
                             int32_t dtype, const fastar_cache* cache, const void* k_cur,
                             const void* v_cur, const uint16_t* kcur_ids, int32_t Ncur, int32_t P,
                             int32_t tables, float scale, const void* out, int32_t out_dtype,
                             const int32_t* best, const float* best_cos, size_t* need) {
    if (!dtype_ok(dtype) || !dtype_ok(out_dtype)) return FASTAR_EDTYPE;
    if (H < 0 || Nq < 0 || Ncur < 0 || !std::isfinite(scale) || !(scale > 0.f)) return FASTAR_EINVAL;
    if (!d_ok(d) || !planes_ok(P) || !tables_ok(P, tables)) return FASTAR_ESHAPE;
    if (cache && (cache->H != H || cache->d != d)) return FASTAR_ESHAPE;
    if (cache && cache->dtype != dtype) return FASTAR_EDTYPE;
    if (!cache_ok(cache, H, d, dtype)) return FASTAR_EINVAL;
    const long long HQ = static_cast<long long>(H) * Nq, HC = static_cast<long long>(H) * Ncur;
    const int cap = cache ? cache->cap : 0;
    if (!fits_i32(HQ * d) || !fits_i32(HC * d) || !fits_i32(static_cast<long long>(H) * (cap + static_cast<long long>(Ncur))))
        return FASTAR_EINVAL;
    if (!head_bytes_ok(cap, d, dtype) || !head_bytes_ok(Ncur, d, dtype)) return FASTAR_EINVAL;
    if (!tensor_ok(q, HQ * d) || !small_ok(q_ids, HQ) || !tensor_ok(out, HQ * d)) return FASTAR_EINVAL;
    if (!tensor_ok(k_cur, HC * d) || !tensor_ok(v_cur, HC * d) || !small_ok(kcur_ids, HC))
        return FASTAR_EINVAL;
    if ((best == nullptr) != (best_cos == nullptr)) return FASTAR_EINVAL;
    if (best && cache && H > 0 && cap > 0 && !cache->knorm) return FASTAR_EINVAL;
    if (tables > 1 && cache && H > 0 && cap > 0 && !cache->ids) return FASTAR_EINVAL;
    *need = tables > 1 ? fastar_annsa_multi_workspace(H, Nq, cap, Ncur, d, P, tables)
                       : fastar_annsa_workspace(H, Nq, cap, Ncur, P);
    return FASTAR_OK;
}

fastar_status annsa_impl(const void* q, const uint16_t* q_ids, int32_t H, int32_t Nq, int32_t d,
                         int32_t dtype, const fastar_cache* cache, const void* k_cur, const void* v_cur,
                         const uint16_t* kcur_ids, int32_t Ncur, int32_t P, int32_t tables, float scale,
                         void* out, int32_t out_dtype, float* lse, int32_t* best, float* best_cos,
                         void* ws, size_t ws_bytes, void* stream) {
    size_t need = 0;
    const fastar_status vs = annsa_validate(q, q_ids, H, Nq, d, dtype, cache, k_cur, v_cur, kcur_ids,
                                            Ncur, P, tables, scale, out, out_dtype, best, best_cos, &need);
    if (vs != FASTAR_OK) return vs;
    if (ws_bytes < need || (need > 0 && !ws)) return FASTAR_EWORKSPACE;
    if (static_cast<long long>(H) * Nq == 0) return FASTAR_OK;
    const int cap = cache ? cache->cap : 0;

    hipStream_t s = static_cast<hipStream_t>(stream);
    Carver c(ws);
    AnnsaWs w = carve_annsa(c, H, Nq, cap, Ncur, P, tables);
    StateWs st = carve_state(c, H, Nq, d, tables);
    // Buckets averaging kQTileWide queries or more take the wide kernel
    // (256-query items), when no search, group sizes or tables are asked for;
    // the item table, sized for 64-query items, holds the fewer wide ones.
    const bool bias = cache && cache->count && cap > 0;
    const bool wide = tables == 1 && !best && !bias && (dtype == FASTAR_BF16 || d == 64) &&
                      (static_cast<long long>(kQTileWide) << P) <= Nq;
    w.it[0].qtile = wide ? kQTileWide : kQTile;
    // every table's (queries, keys) pair sorted in one launch pair; table t
    // groups by id field t (bits tP .. tP+P-1)
    IdSet sets[2 * FASTAR_MAX_TABLES];
    SortBufs bufs[2 * FASTAR_MAX_TABLES];
    for (int t = 0; t < tables; ++t) {
        IdSet& qs = sets[2 * t];
        IdSet& ks = sets[2 * t + 1];
        qs.shift = ks.shift = t * P;
        qs.a = q_ids;
        qs.a_stride = Nq;
        qs.a_fixed = Nq;
        if (cache) {
            ks.a = cache->ids;
            ks.a_stride = cap;
            ks.a_nvalid = cache->n_valid;
            ks.a_cap = cap;
        }
        ks.b = kcur_ids;
        ks.b_stride = Ncur;
        ks.nb = Ncur;
        bufs[2 * t] = w.q[t];
        bufs[2 * t + 1] = w.k[t];
    }
    hipError_t e = launch_bucket_sort(H, P, 2 * tables, sets, bufs, w.it, tables, s);
    if (e != hipSuccess) return FASTAR_EHIP;
    AttnParams p;
    p.q = q;
    p.Nq = Nq;
    p.ka = cache ? cache->k : k_cur;
    p.va = cache ? cache->v : v_cur;
    p.a_rows = cap;
    p.kb = k_cur;
    p.vb = v_cur;
    p.b_rows = Ncur;
    p.n_valid = cache ? cache->n_valid : nullptr;
    p.cap = cap;
    p.out = out;
    p.lse = lse;
    p.best = best;
    p.bcos = best_cos;
    p.knorm = cache ? cache->knorm : nullptr;
    p.kcount = cache ? cache->count : nullptr;
    p.scale_log2 = scale * 1.4426950408889634f;
    p.tables = tables;
    p.wide = wide ? 1 : 0;
    p.fbits = P;
    p.q_ids = q_ids;
    p.ida = cache ? cache->ids : nullptr;
    p.idb = kcur_ids;
    p.st_o = st.o;
    p.st_m = st.m;
    p.st_l = st.l;
    p.st_bc = st.bc;
    p.st_bs = st.bs;
    // one attention launch per table, each resuming the previous one's state
    for (int t = 0; t < tables; ++t) {
        p.qperm = w.q[t].perm;
        p.qperm_stride = w.q[t].perm_stride;
        p.kperm = w.k[t].perm;
        p.kperm_stride = w.k[t].perm_stride;
        p.items = w.it[t].items;
        p.max_items = w.it[t].max_items;
        p.table = t;
        e = launch_attn(MODE_SA, dtype == FASTAR_BF16, d, out_dtype == FASTAR_BF16, H, p, s);
        if (e != hipSuccess) return FASTAR_EHIP;
    }
    return FASTAR_OK;
}

}  // namespace fastar

extern "C" {

fastar_status fastar_annsa_forward(const void* q, const uint16_t* q_ids, int32_t H, int32_t Nq,
                                   int32_t d, int32_t dtype, const fastar_cache* cache,
                                   const void* k_cur, const void* v_cur, const uint16_t* kcur_ids,
                                   int32_t Ncur, int32_t P, float scale, void* out,
                                   int32_t out_dtype, float* lse, int32_t* best, float* best_cos,
                                   void* ws, size_t ws_bytes, void* stream) {
    return annsa_impl(q, q_ids, H, Nq, d, dtype, cache, k_cur, v_cur, kcur_ids, Ncur, P, 1, scale, out,
                      out_dtype, lse, best, best_cos, ws, ws_bytes, stream);
}

fastar_status fastar_annsa_multi_forward(const void* q, const uint16_t* q_ids, int32_t H, int32_t Nq,
                                         int32_t d, int32_t dtype, const fastar_cache* cache,
                                         const void* k_cur, const void* v_cur,
                                         const uint16_t* kcur_ids, int32_t Ncur, int32_t P,
                                         int32_t tables, float scale, void* out, int32_t out_dtype,
                                         float* lse, int32_t* best, float* best_cos, void* ws,
                                         size_t ws_bytes, void* stream) {
    return annsa_impl(q, q_ids, H, Nq, d, dtype, cache, k_cur, v_cur, kcur_ids, Ncur, P, tables, scale,
                      out, out_dtype, lse, best, best_cos, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ AnnCA
size_t fastar_annca_workspace(int32_t H, int32_t Nq, int32_t frame_len, int32_t L, int32_t P) {
    if (H < 0 || Nq < 0 || L < 0 || frame_len <= 0 || !planes_ok(P)) return 0;
    if (L <= kCaFusedMaxL) return 0;          // the attention blocks select the prompt keys
    Carver c(nullptr);
    carve_annca(c, H, Nq / frame_len, L);
    return c.off;
}

fastar_status fastar_annca_forward(const void* q, const uint16_t* q_ids, int32_t H, int32_t Nq,
                                   int32_t frame_len, int32_t d, int32_t dtype, const void* kp,
                                   const void* vp, const uint16_t* kp_ids, int32_t L, int32_t P,
                                   float scale, void* out, int32_t out_dtype, uint8_t* keep,
                                   int32_t* keep_count, void* ws, size_t ws_bytes, void* stream) {
    if (!dtype_ok(dtype) || !dtype_ok(out_dtype)) return FASTAR_EDTYPE;
    if (H < 0 || Nq < 0 || L < 0 || !std::isfinite(scale) || !(scale > 0.f)) return FASTAR_EINVAL;
    if (!d_ok(d) || !planes_ok(P) || frame_len <= 0 || Nq % frame_len != 0) return FASTAR_ESHAPE;
    const long long HQ = static_cast<long long>(H) * Nq, HL = static_cast<long long>(H) * L;
    const int F = Nq / frame_len;
    if (!fits_i32(HQ * d) || !fits_i32(HL * d) || !fits_i32(static_cast<long long>(H) * F * L))
        return FASTAR_EINVAL;
    if (!head_bytes_ok(L, d, dtype)) return FASTAR_EINVAL;
    if (!tensor_ok(q, HQ * d) || !small_ok(q_ids, HQ) || !tensor_ok(out, HQ * d)) return FASTAR_EINVAL;
    if (!tensor_ok(kp, HL * d) || !tensor_ok(vp, HL * d) || !small_ok(kp_ids, HL)) return FASTAR_EINVAL;
    const size_t need = fastar_annca_workspace(H, Nq, frame_len, L, P);
    if (ws_bytes < need || (need > 0 && !ws)) return FASTAR_EWORKSPACE;
    if (HQ == 0) return FASTAR_OK;

    hipStream_t s = static_cast<hipStream_t>(stream);
    AttnParams p;
    if (L <= kCaFusedMaxL) {
        // one launch: each block builds its frame's kept list in LDS
        p.ca_fused = 1;
        p.q_ids = q_ids;
        p.ca_kp_ids = kp_ids;
        p.ca_buckets = 1 << P;
        p.ca_keep = keep;
        p.ca_keep_count = keep_count;
    } else {
        Carver c(ws);
        AnncaWs w = carve_annca(c, H, F, L);
        hipError_t e = launch_annca_select(q_ids, kp_ids, H, Nq, frame_len, L, P, w.idx, w.cnt, keep,
                                           keep_count, s);
        if (e != hipSuccess) return FASTAR_EHIP;
        p.ca_idx = w.idx;
        p.ca_cnt = w.cnt;
    }
    p.q = q;
    p.Nq = Nq;
    p.ka = kp;
    p.va = vp;
    p.a_rows = L;
    p.frame_len = frame_len;
    p.F = F;
    p.L = L;
    p.out = out;
    p.scale_log2 = scale * 1.4426950408889634f;
    return hip_status(launch_attn(MODE_CA, dtype == FASTAR_BF16, d, out_dtype == FASTAR_BF16, H, p, s));
}

// ------------------------------------------------------------------ TempCache
size_t fastar_tempcache_workspace(int32_t H, int32_t N, int32_t cap, int32_t P) {
    if (H < 0 || N < 0 || cap < 0 || !planes_ok(P)) return 0;
    Carver c(nullptr);
    carve_tc(c, H, N, cap, P);
    return c.off;
}

fastar_status fastar_tempcache_order(const fastar_cache* cache, int32_t N, int32_t* order, void* stream) {
    if (!cache) return FASTAR_EINVAL;
    const int H = cache->H, cap = cache->cap;
    if (H < 0 || N < 0 || cap < 0) return FASTAR_EINVAL;
    if (N > cap) return FASTAR_ECAPACITY;
    const long long HN = static_cast<long long>(H) * N;
    if (H > 0 && (!cache->n_valid || (cap > 0 && !cache->ts))) return FASTAR_EINVAL;
    if (!fits_i32(HN) || !small_ok(order, HN)) return FASTAR_EINVAL;
    if (HN == 0) return FASTAR_OK;
    return launch_tc_order(cache->ts, cache->n_valid, H, cap, N, order, static_cast<hipStream_t>(stream)) ==
                   hipSuccess
               ? FASTAR_OK
               : FASTAR_EHIP;
}

fastar_status fastar_tempcache_update(const fastar_cache* cache, const void* q,
                                      const uint16_t* q_ids, const void* k_cur, const void* v_cur,
                                      const uint16_t* kcur_ids, int32_t N, int32_t P, float tau,
                                      int32_t step, const int32_t* best_in, const float* cos_in,
                                      const int32_t* order_in, int32_t* best, float* best_cos,
                                      int32_t* dest, int32_t* evicted, int32_t* counts, void* ws,
                                      size_t ws_bytes, void* stream) {
    if (!cache) return FASTAR_EINVAL;
    const int H = cache->H, d = cache->d, dtype = cache->dtype, cap = cache->cap;
    if (!dtype_ok(dtype)) return FASTAR_EDTYPE;
    if (H < 0 || N < 0 || cap < 0 || std::isnan(tau)) return FASTAR_EINVAL;
    if (!d_ok(d) || !planes_ok(P)) return FASTAR_ESHAPE;
    if (!cache_ok(cache, H, d, dtype)) return FASTAR_EINVAL;
    if (H > 0 && (!cache->ids || !cache->ts || !cache->n_valid ||
                  (cap > 0 && (!cache->k || !cache->v || !cache->knorm))))
        return FASTAR_EINVAL;
    if ((best_in == nullptr) != (cos_in == nullptr)) return FASTAR_EINVAL;
    if (N > cap) return FASTAR_ECAPACITY;
    const long long HN = static_cast<long long>(H) * N;
    if (!fits_i32(HN * d) || !head_bytes_ok(cap, d, dtype)) return FASTAR_EINVAL;
    if (!tensor_ok(q, HN * d) || !small_ok(q_ids, HN) || !tensor_ok(k_cur, HN * d) ||
        !tensor_ok(v_cur, HN * d) || !small_ok(kcur_ids, HN))
        return FASTAR_EINVAL;
    const size_t need = fastar_tempcache_workspace(H, N, cap, P);
    if (ws_bytes < need || (need > 0 && !ws)) return FASTAR_EWORKSPACE;
    if (H == 0) return FASTAR_OK;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool bf = dtype == FASTAR_BF16;
    Carver c(ws);
    TcWs w = carve_tc(c, H, N, cap, P);
    hipError_t e = hipSuccess;

    const int32_t* bestp;
    const float* cosp;
    if (best_in) {
        bestp = best_in;
        cosp = cos_in;
        if (best && HN > 0)
            e = hipMemcpyAsync(best, best_in, HN * sizeof(int32_t), hipMemcpyDeviceToDevice, s);
        if (e == hipSuccess && best_cos && HN > 0)
            e = hipMemcpyAsync(best_cos, cos_in, HN * sizeof(float), hipMemcpyDeviceToDevice, s);
        if (e != hipSuccess) return FASTAR_EHIP;
    } else {
        int32_t* bo = best ? best : w.best;
        float* co = best_cos ? best_cos : w.cosv;
        bestp = bo;
        cosp = co;
        IdSet sets[2];
        sets[0].a = q_ids;
        sets[0].a_stride = N;
        sets[0].a_fixed = N;
        sets[1].a = cache->ids;
        sets[1].a_stride = cap;
        sets[1].a_nvalid = cache->n_valid;
        sets[1].a_cap = cap;
        SortBufs bufs[2] = {w.q, w.k};
        e = launch_bucket_sort(H, P, 2, sets, bufs, &w.it, 1, s);
        if (e != hipSuccess) return FASTAR_EHIP;
        AttnParams p;
        p.q = q;
        p.Nq = N;
        p.ka = cache->k;
        p.a_rows = cap;
        p.n_valid = cache->n_valid;
        p.cap = cap;
        p.qperm = w.q.perm;
        p.qperm_stride = w.q.perm_stride;
        p.kperm = w.k.perm;
        p.kperm_stride = w.k.perm_stride;
        p.items = w.it.items;
        p.max_items = w.it.max_items;
        p.knorm = cache->knorm;
        p.best = bo;
        p.bcos = co;
        e = launch_attn(MODE_TOP1, bf, d, false, H, p, s);
        if (e != hipSuccess) return FASTAR_EHIP;
    }

    TcSelectParams sp;
    sp.best = bestp;
    sp.cosv = cosp;
    sp.claim = w.claim;
    sp.refreshed = w.refreshed;
    sp.ts = cache->ts;
    sp.n_valid = cache->n_valid;
    sp.upos = w.upos;
    sp.ev = w.ev;
    sp.dest = dest ? dest : w.dest;
    sp.evicted = evicted;
    sp.counts = counts;
    sp.order = order_in;
    const bool merge = cache->count != nullptr && cap > 0;
    sp.grp_cnt = merge ? w.grp_cnt : nullptr;
    sp.grp_off = merge ? w.grp_off : nullptr;
    sp.grp_mem = merge ? w.grp_mem : nullptr;
    sp.grp_pos = merge ? w.grp_pos : nullptr;
    sp.H = H;
    sp.N = N;
    sp.cap = cap;
    sp.tau = tau;
    e = launch_tc_select(sp, s);
    if (e != hipSuccess) return FASTAR_EHIP;
    if (merge)
        return hip_status(launch_tc_merge_scatter(bf, d, H, N, cap, sp.dest, sp.grp_cnt, sp.grp_off,
                                                  sp.grp_mem, k_cur, v_cur, kcur_ids, step, cache->k,
                                                  cache->v, cache->ids, cache->ts, cache->knorm,
                                                  cache->count, s));
    return hip_status(launch_tc_scatter(bf, d, H, N, cap, sp.dest, k_cur, v_cur, kcur_ids, step,
                                        cache->k, cache->v, cache->ids, cache->ts, cache->knorm, s));
}

// ------------------------------------------------------------------ timer
fastar_status fastar_timer_start(void) {
    g_recs.clear();
    g_pool_used = 0;
    g_timer_on = true;
    return FASTAR_OK;
}

int32_t fastar_timer_stop(fastar_kernel_time* out, int32_t max) {
    g_timer_on = false;
    g_pending = false;
    std::vector<fastar_kernel_time> agg;
    for (const TimerRec& r : g_recs) {
        float ms = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess) continue;
        if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) continue;
        size_t i = 0;
        for (; i < agg.size(); ++i)
            if (std::strncmp(agg[i].name, r.name, sizeof(agg[i].name)) == 0) break;
        if (i == agg.size()) {
            fastar_kernel_time k;
            std::memset(&k, 0, sizeof(k));
            std::strncpy(k.name, r.name, sizeof(k.name) - 1);
            agg.push_back(k);
        }
        agg[i].launches += 1;
        agg[i].total_ms += ms;
    }
    g_recs.clear();
    g_pool_used = 0;
    const int n = static_cast<int>(agg.size());
    for (int i = 0; i < n && i < max && out; ++i) out[i] = agg[i];
    return n;
}

}  // extern "C"
