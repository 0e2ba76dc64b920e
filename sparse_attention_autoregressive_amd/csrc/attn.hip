// Gathered block attention on the matrix cores, three uses:
//
//  MODE_SA   AnnSA: work items are (head, bucket, 64-query slice).  Queries are
//            the bucket's current-chunk queries, keys the bucket's members of
//            [cache slots ; current chunk] (FAST-AR blog, "3. AnnSA"; summary,
//            "2. Core Components" C).  Softmax attention + log-sum-exp.  With
//            SEARCH the same pass also finds each query's most similar cached
//            key (TempCache's top-1, blog "1. TempCache"; summary A): those
//            keys are exactly the cached members of the query's bucket, whose
//            dot products the attention computes anyway.
//  MODE_CA   AnnCA: one block per (head, frame, 64 or 128 consecutive queries); keys
//            are the frame's kept prompt tokens (blog, "2. AnnCA"; summary B).
//  MODE_TOP1 TempCache search alone: the SA items over cached keys only, no
//            softmax; each query keeps its best cosine and slot.
//
// Layout of the work on one 64-query item (256 threads = 4 waves, wave w owns
// the item's queries 16w..16w+15; lane l serves query l%16 and "lane group"
// g = l/16):
//  * scores are computed transposed, S^T = K Q^T, so that MFMA's output layout
//    (lane holds rows 4g..4g+3 of column l%16) gives every lane a single query
//    and four keys per 16-key block: the row max / sum of the online softmax
//    then need only two cross-lane steps (lanes l, l^16, l^32, l^48), and the
//    probabilities are already laid out as the B operand of O^T = V^T P^T.
//  * K and V tiles of 64 rows sit row-major in LDS (16-byte stores, rows
//    padded).  K fragments (A operand of S^T) are 16 contiguous bytes per lane.
//    The bf16 V^T fragments come from gfx950's LDS transpose read
//    (ds_read_b64_tr_b16): within each 16-lane group, lane i receives element
//    i%4 of the 8-byte chunks addressed by lanes 4k + i/4 (k = 0..3), so when
//    lane j points at V[key0 + j/4][d0 + 4(j%4)] lane i gets dim d0+i of keys
//    key0..key0+3.  Two such reads give lane group g the keys
//    {4g..4g+3, 16+4g..16+4g+3} of a 32-key group -- exactly the keys its
//    probabilities cover in the B operand.  For fp32 (16x16x4 MFMA) V is read
//    row-major.
//  * The item's key indices are staged in LDS; K/V rows are gathered with
//    16-byte loads (16 lanes cover one 256-byte bf16 row) into two register
//    stages, so two tiles are in flight while a third is computed on.
//  * The search uses the cached keys' norms kept in the cache, so a cosine is
//    one product per (query, key): dot * (1/|k|), times 1/|q| at the end.
//  * MULTI (multi-table AnnSA; blog, "3. AnnSA": a token may fall in several
//    buckets): ids hold one P-bit field per table and the host launches the
//    kernel once per table over that table's items.  A pair whose ids agree
//    in an earlier table's field was counted there and is masked here, so each
//    key of a query's union of buckets counts once; each query's online
//    softmax (unnormalised O, running max and sum) and search state carry over
//    between the launches through the workspace, and the last launch
//    normalises.  Each key's id travels with its tile like the norms.
//  * BIAS (AnnSA over a mean-merged cache; summary, "2. Core Components" A,
//    Lemma 5.1): a cached slot that stands for m tokens adds ln m to its
//    logits.  The group sizes travel with the tile like the norms, one load
//    per thread, and become a per-key score offset ln(m) / scale in LDS.
//
// Every use launches one block per item, heads fastest in the launch order;
// SA / TOP1 items come from a table the bucket sort writes with the longest
// key lists first, so the largest buckets never form the tail of the launch.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

#ifndef CA_WAVES
#define CA_WAVES 4
#endif
#ifndef CA_GROUPS
#define CA_GROUPS 2              // 16-query groups per AnnCA wave
#endif
#ifndef CA_XCD
#define CA_XCD 1                 // AnnCA blocks of one (head, frame) on one XCD
#endif
#ifndef SA_XCD_RUN
#define SA_XCD_RUN 4             // AnnSA work items dealt to the XCDs in runs of this many (1: in turn)
#endif

namespace fastar {

namespace {

constexpr int KT = 64;            // keys per LDS tile
constexpr int KCH = 1024;         // key indices staged in LDS at a time
constexpr float kNegInf = -__builtin_huge_valf();
// Online softmax: the exponent's reference (a running maximum) moves only when
// a score passes it by more than this many powers of two (log2 units; 0
// rescales whenever the maximum grows).
#ifndef SOFTMAX_RESCALE_LOG2
#define SOFTMAX_RESCALE_LOG2 8
#endif
constexpr float kRescaleLog2 = SOFTMAX_RESCALE_LOG2;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// 4 bf16 of V^T through the LDS transpose read (see the header comment).
__device__ __forceinline__ v4i16 lds_read_tr(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(const_cast<void*>(p)));
}

template <typename T, int D, int MODE, int NT>
struct Tile {
    static constexpr bool BF = sizeof(T) == 2;
    static constexpr bool HAS_V = MODE != MODE_TOP1;
    static constexpr int EPC = 16 / sizeof(T);          // elements per 16-byte chunk
    static constexpr int CPR = D / EPC;                 // chunks per row
    // Thread u of NT gathers chunk u % CPR of the E rows (u / CPR) * E + e.
    static constexpr int E = KT * CPR / NT;
    static_assert(E >= 1 && KT * CPR % NT == 0, "tile split");
    // Padded rows.  K rows step 4 banks (mod 64), so the 16 rows one K-fragment
    // read touches cover all 64 banks.  bf16 V rows step 8 banks, so the 4 rows
    // x 4 8-byte columns of a transpose read (and the 4 lane groups, 4 rows
    // apart) fall on distinct banks.
    static constexpr int STRK = D + EPC;
    static constexpr int STRV = BF ? D + 2 * EPC : D + EPC;
    static constexpr int ROWB = D * static_cast<int>(sizeof(T));   // bytes per global row
    static constexpr int NDB = D / 16;                  // 16-wide output blocks
    static constexpr int NKS = BF ? D / 32 : D / 4;     // k-steps of S^T
};

// The pieces every kernel below is built from.
template <typename T, int D, int MODE, bool SEARCH, int NT, bool BIAS = false, bool MULTI = false>
struct Blk {
    static_assert(!BIAS || MODE == MODE_SA, "group-size offsets are AnnSA's");
    static_assert(!MULTI || MODE == MODE_SA, "tables are AnnSA's");
    static constexpr bool SLOTS = SEARCH || BIAS;     // the tile's key indices go to LDS
    using TL = Tile<T, D, MODE, NT>;
    static constexpr bool BF = TL::BF, HAS_V = TL::HAS_V;
    static constexpr int E = TL::E, CPR = TL::CPR, EPC = TL::EPC;
    static constexpr int STRK = TL::STRK, STRV = TL::STRV, ROWB = TL::ROWB;
    static constexpr int NDB = TL::NDB, NKS = TL::NKS;
    // AnnCA (no lse output) lets the softmax reference lag (kRescaleLog2) and,
    // with bf16 products, sums the probabilities as rounded for the PV
    // product; AnnSA keeps the exact running maximum and fp32 sums, so that
    // its lse carries no bf16 rounding.
    static constexpr bool LAZY = MODE == MODE_CA;
    static constexpr bool RSUM = LAZY && BF;

    // B operand of S^T: lane holds Q[query l%16][k-slice of group g].
    struct QF {
        bf16x8_t b[BF ? NKS : 1];
        float f[BF ? 1 : NKS];
        float inv;                  // 1/|q| (search only)
    };
    // One 64-key tile between its global gather and its LDS store.  (Its key
    // slots, for the search, wait in an LDS array of the stage, ``slots``.)
    struct Stage {
        u32x4 k[E];
        u32x4 v[HAS_V ? E : 1];
        float kn;                   // search: the norm of row (u / CPR) * E + u % CPR (u % CPR < E)
        int kc;                     // bias: that row's group size
        int kq;                     // multi-table: that row's id
        int* slots;
    };
    // Running state of one query (per lane; the four lane groups of a query
    // hold disjoint keys and are merged at the end).
    struct Acc {
        f32x4 o[HAS_V ? NDB : 1];
        float m, l;                 // softmax: reference maximum (raw score units), sum
        float bc;                   // search: best dot/|k|
        int bs;                     //         and its slot
        __device__ __forceinline__ void reset() {
#pragma unroll
            for (int i = 0; i < (HAS_V ? NDB : 1); ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            m = kNegInf;
            l = 0.f;
            bc = kNegInf;
            bs = 0x7FFFFFFF;
        }
    };
    struct Smem {
        T* Ks;
        T* Vs;
        int* kslot;
        float* kinv;
        float* kbias;
        int* kid;
    };
    // Where one head's keys live: index j < na is row j of (ka, va), else row
    // j - na of (kb, vb).  kn holds the cached keys' norms.
    struct Src {
        const T* ka;
        const T* va;
        const T* kb;
        const T* vb;
        const float* kn;
        const int32_t* kcnt;
        const uint16_t* ida;
        const uint16_t* idb;
        int na;
    };

    // Issues the loads of a query row's fragments (``row`` null: a padding lane).
    static __device__ __forceinline__ void load_q(QF& q, const T* row, int g) {
        if constexpr (BF) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                u32x4 r = {0u, 0u, 0u, 0u};
                if (row) r = *reinterpret_cast<const u32x4*>(row + ks * 32 + 8 * g);
                q.b[ks] = __builtin_bit_cast(bf16x8_t, r);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) q.f[ks] = row ? reinterpret_cast<const float*>(row)[ks * 4 + g] : 0.f;
        }
    }
    // The same from a row that is always there: no branch, so the compiler
    // can count these loads when a later wait needs only older ones.
    static __device__ __forceinline__ void load_q_row(QF& q, const T* row, int g) {
        if constexpr (BF) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                q.b[ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(row + ks * 32 + 8 * g));
        } else {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) q.f[ks] = reinterpret_cast<const float*>(row)[ks * 4 + g];
        }
    }
    // 1/|q| from the fragments (all lanes of the wave take part).
    static __device__ __forceinline__ void finish_q(QF& q) {
        if constexpr (!SEARCH) return;
        float qsq = 0.f;
        if constexpr (BF) {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const u32x4 r = __builtin_bit_cast(u32x4, q.b[ks]);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float lo = __uint_as_float(r[i] << 16), hi = __uint_as_float(r[i] & 0xFFFF0000u);
                    qsq = __builtin_fmaf(lo, lo, qsq);
                    qsq = __builtin_fmaf(hi, hi, qsq);
                }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) qsq = __builtin_fmaf(q.f[ks], q.f[ks], qsq);
        }
        qsq += __shfl_xor(qsq, 16);
        qsq += __shfl_xor(qsq, 32);
        const float qn = __builtin_sqrtf(qsq);
        q.inv = qn > 0.f ? 1.f / qn : 0.f;
    }

    // Gathers tile ``tile`` of the key list staged in ``kidx``.  Rows of a tile
    // come from the cache part or the current chunk; the key list holds cached
    // keys first, so at most one tile per item mixes the two, and every other
    // tile gathers from one base pointer held in scalar registers with a
    // 32-bit byte offset per row.
    template <bool LK = true, bool LV = true>
    static __device__ __forceinline__ void load_tile(Stage& S, const int* kidx, int tile, const Src& sr,
                                                     int tid) {
        int jf = 0, jl = 0;
        if constexpr (MODE == MODE_SA) {
            jf = __builtin_amdgcn_readfirstlane(kidx[(tile * KT) % KCH]);
            jl = __builtin_amdgcn_readfirstlane(kidx[(tile * KT + KT - 1) % KCH]);
        }
        const bool all_a = MODE != MODE_SA || jl < sr.na;        // scalar
        const bool all_b = MODE == MODE_SA && jf >= sr.na;
        const char* kbase = reinterpret_cast<const char*>(all_a ? sr.ka : sr.kb);
        const char* vbase = HAS_V ? reinterpret_cast<const char*>(all_a ? sr.va : sr.vb) : nullptr;
        const int sub = all_a ? 0 : sr.na;
        const int chunk = tid % CPR, rb = tid / CPR;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int row = rb * E + e;
            const int j = kidx[(tile * KT + row) % KCH];
            if (all_a || all_b) {
                const uint32_t off = static_cast<uint32_t>(j - sub) * ROWB + chunk * 16;
                if constexpr (LK) S.k[e] = *reinterpret_cast<const u32x4*>(kbase + off);
                if constexpr (HAS_V && LV) S.v[e] = *reinterpret_cast<const u32x4*>(vbase + off);
            } else {
                const bool from_a = j < sr.na;
                const uint32_t off = static_cast<uint32_t>(from_a ? j : j - sr.na) * ROWB + chunk * 16;
                if constexpr (LK)
                    S.k[e] = *reinterpret_cast<const u32x4*>(
                        reinterpret_cast<const char*>(from_a ? sr.ka : sr.kb) + off);
                if constexpr (HAS_V && LV)
                    S.v[e] = *reinterpret_cast<const u32x4*>(
                        reinterpret_cast<const char*>(from_a ? sr.va : sr.vb) + off);
            }
        }
        if constexpr (!LK) return;
        if constexpr (SLOTS) {
            // One norm (and group size) per thread: lanes u % CPR = e < E
            // take row rb*E + e (the others repeat row rb*E + E-1), so a tile
            // costs one load per thread, issued without a branch; current-
            // chunk keys read a clamped cached index and are masked at the
            // store.
            const int row = rb * E + (chunk < E ? chunk : E - 1);
            const int j = kidx[(tile * KT + row) % KCH];
            const int jc = MODE != MODE_SA || j < sr.na ? j : sr.na - 1;
            if constexpr (SEARCH) {
                if (MODE != MODE_SA || sr.na > 0)                  // uniform
                    S.kn = sr.kn[jc];
                else
                    S.kn = 0.f;
            }
            if constexpr (BIAS) S.kc = sr.na > 0 ? sr.kcnt[jc] : 1;
            S.slots[row] = j;
        }
        if constexpr (MULTI) {
            const int row = rb * E + (chunk < E ? chunk : E - 1);
            const int j = kidx[(tile * KT + row) % KCH];
            S.kq = *(j < sr.na ? sr.ida + j : sr.idb + (j - sr.na));
        }
    }

    // ``inv_c`` = 1 / (scale * log2 e): a group size m becomes the raw-score
    // offset log2(m) * inv_c = ln(m) / scale.
    // ``SV``: the stage whose V part is stored (the K stage itself, or a
    // separate V stage in the split pipeline).
    static __device__ __forceinline__ void store_tile(const Stage& S, const Smem& sm, int na, int tid,
                                                      float inv_c, const Stage* SV = nullptr) {
        const int chunk = tid % CPR, rb = tid / CPR;
        const Stage& V = SV ? *SV : S;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int row = rb * E + e;
            *reinterpret_cast<u32x4*>(&sm.Ks[row * STRK + chunk * EPC]) = S.k[e];
            if constexpr (HAS_V) *reinterpret_cast<u32x4*>(&sm.Vs[row * STRV + chunk * EPC]) = V.v[e];
        }
        if constexpr (SLOTS) {
            if (chunk < E) {
                const int row = rb * E + chunk;
                const int j = S.slots[row];
                if constexpr (SEARCH) {
                    sm.kslot[row] = j;
                    sm.kinv[row] = (MODE == MODE_TOP1 || j < na) && S.kn > 0.f ? __builtin_amdgcn_rcpf(S.kn) : 0.f;
                }
                if constexpr (BIAS)
                    sm.kbias[row] = j < na && S.kc > 1
                                        ? __builtin_amdgcn_logf(static_cast<float>(S.kc)) * inv_c
                                        : 0.f;
            }
        }
        if constexpr (MULTI)
            if (chunk < E) sm.kid[rb * E + chunk] = S.kq;
    }

    // Online softmax of one 16-query group over a 64-key tile (one query per
    // lane): masks the keys past nk, updates the reference maximum, sum and
    // output scale, and leaves the probabilities in ``s``.  The reference m is
    // kept in raw score units; the scale folds into the exponent:
    // p = 2^(s*c - m*c), c = scale * log2(e) > 0.  m follows the running
    // maximum lazily: it moves (and the sum and output are rescaled) only on
    // a query's first keys or when the tile's maximum passes it by more than
    // kRescaleLog2 in the exponent, so p <= 2^kRescaleLog2 and most tiles skip
    // the rescale (LAZY; otherwise m is the running maximum itself).  Output,
    // sum and lse share the one reference, so the result is the softmax's up
    // to rounding.  With RSUM the caller sums the probabilities as rounded for
    // the PV product (bf16_sum8), so that the normaliser matches the
    // numerator: with a lagging reference the largest p is not 1, and its
    // rounding would otherwise show in the output.
    // The maximum of x over lanes i, i^16, i^32 and i^48 -- the four lane
    // groups that hold one query's keys.  Each lane swap (gfx950's
    // v_permlane32_swap / v_permlane16_swap) leaves x of the lane and of its
    // partner in the two results, in the VALU, without an LDS round trip.
    // Larger of two scores.  gfx950's NaN-propagating maximum takes its
    // operands as they are, where fmaxf first canonicalises each operand not
    // known to be canonical (MFMA results, lane swaps): one more VALU op per
    // operand.  Scores hold no NaN (masked keys are -inf), so the two agree.
    static __device__ __forceinline__ float smax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
    static __device__ __forceinline__ float max_over_groups(float x) {
        const uint32_t u = __float_as_uint(x);
        const auto a32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        const float y = smax(__uint_as_float(a32[0]), __uint_as_float(a32[1]));
        const uint32_t v = __float_as_uint(y);
        const auto a16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return smax(__uint_as_float(a16[0]), __uint_as_float(a16[1]));
    }
    static __device__ __forceinline__ void softmax_update(Acc& a, f32x4 (&s)[4], bool full, int kbase, int nk,
                                                          float scale_log2, int g) {
        if (!full) {
#pragma unroll
            for (int kb4 = 0; kb4 < 4; ++kb4)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (kbase + kb4 * 16 + 4 * g + r >= nk) s[kb4][r] = kNegInf;
        }
        float t[4];
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4) t[kb4] = smax(smax(s[kb4][0], s[kb4][1]), smax(s[kb4][2], s[kb4][3]));
        const float tmax = max_over_groups(smax(smax(t[0], t[1]), smax(t[2], t[3])));
        const float m_new = smax(a.m, tmax);
        const float c = scale_log2;
        const float m_ref = (a.m == kNegInf || (m_new - a.m) * c > (LAZY ? kRescaleLog2 : 0.f)) ? m_new : a.m;
        const float mc = (m_ref == kNegInf) ? 0.f : m_ref * c;
        float psum = 0.f;
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb4][r], c, -mc));
                s[kb4][r] = e;
                if constexpr (!RSUM) psum += e;
            }
        }
        if (__ballot(m_ref > a.m) != 0) {                   // some lane's reference moved
            const float alpha = (a.m == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(a.m, c, -mc));
            a.l *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) a.o[db] *= alpha;
        }
        if constexpr (!RSUM) a.l += psum;
        a.m = m_ref;
    }
    // acc plus the eight bf16 values of ``p`` (exact products with 1, fp32 sums).
    static __device__ __forceinline__ float bf16_sum8(const bf16x8_t& p, float acc) {
        const bf16x2_t ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 0, 1), ones, acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 2, 3), ones, acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 4, 5), ones, acc, false);
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 6, 7), ones, acc, false);
    }

    // One 64-key tile (keys kbase.. of an item with nk keys, the first na of
    // the head's index space cached) against the wave's 16 queries.
    // ``seen``: for multi-table launches, (query id, table, field bits); a pair
    // whose ids agree in a field below ``table`` is masked.
    struct Seen {
        int qid, table, fbits;
    };
    static __device__ __forceinline__ void compute_tile(Acc& a, const QF& q, const Smem& sm, int kbase,
                                                        int nk, int na, float scale_log2, int g, int c16,
                                                        const Seen& seen = Seen{0, 0, 0}) {
        // ---- S^T = K Q^T for the 4 key blocks of the tile
        f32x4 s[4];
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4) {
            s[kb4] = f32x4{0.f, 0.f, 0.f, 0.f};
            const T* krow = &sm.Ks[(kb4 * 16 + c16) * STRK];
            if constexpr (BF) {
                bf16x8_t af[NKS];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    af[ks] = *reinterpret_cast<const bf16x8_t*>(krow + ks * 32 + 8 * g);
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    s[kb4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks], q.b[ks], s[kb4], 0, 0, 0);
            } else {
                float af[NKS];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) af[ks] = reinterpret_cast<const float*>(krow)[ks * 4 + g];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    s[kb4] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[ks], q.f[ks], s[kb4], 0, 0, 0);
            }
        }
        const bool full = kbase + KT <= nk;                    // uniform

        // ---- TempCache search over this tile's cached keys (sorted first, so a
        // tile whose first key is current holds no cached key).  The running
        // best compares dot * (1/|k|); 1/|q| > 0 is applied once at the end.
        if constexpr (SEARCH) {
            if (MODE == MODE_TOP1 || sm.kslot[0] < na) {
                // uniform: a full tile of cached keys needs no per-key masks
                const bool clean = full && (MODE == MODE_TOP1 || sm.kslot[KT - 1] < na);
                auto scan = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
                    for (int kb4 = 0; kb4 < 4; ++kb4) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int sl = sm.kslot[kb4 * 16 + 4 * g + r];
                            const float cs = s[kb4][r] * sm.kinv[kb4 * 16 + 4 * g + r];
                            bool ok = cs > a.bc;
                            if constexpr (decltype(masked)::value)
                                ok = ok && (MODE == MODE_TOP1 || sl < na) &&
                                     kbase + kb4 * 16 + 4 * g + r < nk;
                            a.bc = ok ? cs : a.bc;
                            a.bs = ok ? sl : a.bs;
                        }
                    }
                };
                if (clean) scan(std::false_type{});
                else scan(std::true_type{});
            }
        }

        if constexpr (HAS_V) {
            // ---- multi-table: keys that share the query's bucket in an
            // earlier table were counted by that table's launch (after the
            // search: a repeated key gives the same cosine)
            if constexpr (MULTI) {
                if (seen.table > 0) {                              // uniform
                    const uint32_t fm = (1u << seen.fbits) - 1u;
#pragma unroll
                    for (int kb4 = 0; kb4 < 4; ++kb4) {
                        const int4 kk = *reinterpret_cast<const int4*>(&sm.kid[kb4 * 16 + 4 * g]);
                        const int kv[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const uint32_t x = static_cast<uint32_t>(seen.qid ^ kv[r]);
                            bool dup = false;
                            for (int t = 0; t < seen.table; ++t) dup |= ((x >> (t * seen.fbits)) & fm) == 0u;
                            s[kb4][r] = dup ? kNegInf : s[kb4][r];
                        }
                    }
                }
            }
            // ---- group-size offsets of a mean-merged cache (after the search,
            // which compares plain cosines)
            if constexpr (BIAS) {
#pragma unroll
                for (int kb4 = 0; kb4 < 4; ++kb4) {
                    const float4 b = *reinterpret_cast<const float4*>(&sm.kbias[kb4 * 16 + 4 * g]);
                    s[kb4][0] += b.x;
                    s[kb4][1] += b.y;
                    s[kb4][2] += b.z;
                    s[kb4][3] += b.w;
                }
            }
            softmax_update(a, s, full, kbase, nk, scale_log2, g);

            // ---- O^T += V^T P^T
            if constexpr (BF) {
#pragma unroll
                for (int kg = 0; kg < 2; ++kg) {
                    bf16x8_t pb;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pb[r] = static_cast<__bf16>(s[2 * kg][r]);
                        pb[4 + r] = static_cast<__bf16>(s[2 * kg + 1][r]);
                    }
                    if constexpr (RSUM) a.l = bf16_sum8(pb, a.l);
                    // lane j of group g addresses V[kg*32 + 4g + j/4][db*16 + 4(j%4)]
                    const T* vb0 = &sm.Vs[(kg * 32 + 4 * g + (c16 >> 2)) * STRV + 4 * (c16 & 3)];
                    v4i16 lo[NDB], hi[NDB];
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        lo[db] = lds_read_tr(vb0 + db * 16);
                        hi[db] = lds_read_tr(vb0 + 16 * STRV + db * 16);
                    }
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const bf16x8_t av = __builtin_bit_cast(
                            bf16x8_t, __builtin_shufflevector(lo[db], hi[db], 0, 1, 2, 3, 4, 5, 6, 7));
                        a.o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb, a.o[db], 0, 0, 0);
                    }
                }
            } else {
#pragma unroll
                for (int kb4 = 0; kb4 < 4; ++kb4) {
#pragma unroll
                    for (int st = 0; st < 4; ++st) {
                        const float* vrow = reinterpret_cast<const float*>(&sm.Vs[(kb4 * 16 + 4 * g + st) * STRV]);
#pragma unroll
                        for (int db = 0; db < NDB; ++db)
                            a.o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vrow[db * 16 + c16], s[kb4][st], a.o[db], 0, 0, 0);
                    }
                }
            }
        }
    }

    // NG 16-query groups per wave (AnnCA, wide AnnSA): each K and V fragment
    // read from LDS feeds the MFMAs of every group, so LDS reads per product
    // fall as 1/NG.
    template <int NG>
    static __device__ __forceinline__ void compute_tileg(Acc (&a)[NG], const QF (&q)[NG], const Smem& sm,
                                                         int kbase, int nk, float scale_log2, int g,
                                                         int c16) {
        static_assert(MODE != MODE_TOP1 && !SEARCH && !BIAS && !MULTI,
                      "query groups: AnnCA and plain AnnSA only");
        f32x4 s[NG][4];
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4) {
#pragma unroll
            for (int qg = 0; qg < NG; ++qg) s[qg][kb4] = f32x4{0.f, 0.f, 0.f, 0.f};
            const T* krow = &sm.Ks[(kb4 * 16 + c16) * STRK];
            if constexpr (BF) {
                bf16x8_t af[NKS];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    af[ks] = *reinterpret_cast<const bf16x8_t*>(krow + ks * 32 + 8 * g);
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int qg = 0; qg < NG; ++qg)
                        s[qg][kb4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks], q[qg].b[ks], s[qg][kb4], 0, 0, 0);
            } else {
                float af[NKS];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) af[ks] = reinterpret_cast<const float*>(krow)[ks * 4 + g];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int qg = 0; qg < NG; ++qg)
                        s[qg][kb4] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[ks], q[qg].f[ks], s[qg][kb4], 0, 0, 0);
            }
        }
        const bool full = kbase + KT <= nk;                    // uniform
#pragma unroll
        for (int qg = 0; qg < NG; ++qg) softmax_update(a[qg], s[qg], full, kbase, nk, scale_log2, g);
        if constexpr (BF) {
#pragma unroll
            for (int kg = 0; kg < 2; ++kg) {
                bf16x8_t pb[NG];
#pragma unroll
                for (int qg = 0; qg < NG; ++qg)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        pb[qg][r] = static_cast<__bf16>(s[qg][2 * kg][r]);
                        pb[qg][4 + r] = static_cast<__bf16>(s[qg][2 * kg + 1][r]);
                    }
#pragma unroll
                for (int qg = 0; qg < NG; ++qg)
                    if constexpr (RSUM) a[qg].l = bf16_sum8(pb[qg], a[qg].l);
                const T* vb0 = &sm.Vs[(kg * 32 + 4 * g + (c16 >> 2)) * STRV + 4 * (c16 & 3)];
                v4i16 lo[NDB], hi[NDB];
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    lo[db] = lds_read_tr(vb0 + db * 16);
                    hi[db] = lds_read_tr(vb0 + 16 * STRV + db * 16);
                }
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const bf16x8_t av = __builtin_bit_cast(
                        bf16x8_t, __builtin_shufflevector(lo[db], hi[db], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
                    for (int qg = 0; qg < NG; ++qg)
                        a[qg].o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[qg], a[qg].o[db], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int kb4 = 0; kb4 < 4; ++kb4) {
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const float* vrow = reinterpret_cast<const float*>(&sm.Vs[(kb4 * 16 + 4 * g + st) * STRV]);
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const float vv = vrow[db * 16 + c16];
#pragma unroll
                        for (int qg = 0; qg < NG; ++qg)
                            a[qg].o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv, s[qg][kb4][st], a[qg].o[db], 0, 0, 0);
                    }
                }
            }
        }
    }

    // Merges the four lane groups of each query and writes its results
    // (all lanes of the wave take part in the merge).  Row pointers are those
    // of the lane's query; ``qvalid`` false for padding lanes.
    template <typename OT>
    static __device__ __forceinline__ void finish(Acc& a, const QF& q, bool qvalid, int g, OT* orow,
                                                  float* lse, int32_t* best, float* bcos, float scale_log2) {
        if constexpr (SEARCH) {
#pragma unroll
            for (int off = 16; off <= 32; off <<= 1) {
                const float oc = __shfl_xor(a.bc, off);
                const int os = __shfl_xor(a.bs, off);
                if (oc > a.bc || (oc == a.bc && os < a.bs)) { a.bc = oc; a.bs = os; }
            }
            if (qvalid && g == 0) {
                const bool found = a.bs != 0x7FFFFFFF;
                *best = found ? a.bs : -1;
                *bcos = found ? a.bc * q.inv : kNegInf;
            }
        }
        if constexpr (HAS_V) {
            float l_tot = a.l + __shfl_xor(a.l, 16);
            l_tot += __shfl_xor(l_tot, 32);
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            if (qvalid) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const f32x4 v = a.o[db] * inv;
                    if constexpr (sizeof(OT) == 4) {
                        *reinterpret_cast<f32x4*>(orow + db * 16 + 4 * g) = v;
                    } else {
                        const uint32_t lo = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
                        const uint32_t hi = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
                        *reinterpret_cast<uint2*>(orow + db * 16 + 4 * g) = make_uint2(lo, hi);
                    }
                }
                if (MODE == MODE_SA && lse && g == 0)
                    *lse = l_tot > 0.f ? (a.m * scale_log2 + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f
                                       : kNegInf;
            }
        }
    }

    // Multi-table, every launch but the last: the query's state goes to the
    // workspace instead of the output (the search and sum merged over the four
    // lane groups as in ``finish``; O stays unnormalised).
    static __device__ __forceinline__ void store_state(Acc& a, bool qvalid, int g, size_t qi,
                                                       const AttnParams& p) {
        if constexpr (SEARCH) {
#pragma unroll
            for (int off = 16; off <= 32; off <<= 1) {
                const float oc = __shfl_xor(a.bc, off);
                const int os = __shfl_xor(a.bs, off);
                if (oc > a.bc || (oc == a.bc && os < a.bs)) { a.bc = oc; a.bs = os; }
            }
        }
        float l_tot = a.l + __shfl_xor(a.l, 16);
        l_tot += __shfl_xor(l_tot, 32);
        if (!qvalid) return;
#pragma unroll
        for (int db = 0; db < NDB; ++db) *reinterpret_cast<f32x4*>(p.st_o + qi * D + db * 16 + 4 * g) = a.o[db];
        if (g == 0) {
            p.st_m[qi] = a.m;
            p.st_l[qi] = l_tot;
            if constexpr (SEARCH) {
                p.st_bc[qi] = a.bc;
                p.st_bs[qi] = a.bs;
            }
        }
    }
    // Multi-table, every launch but the first: resume the query's state (the
    // sum enters through lane group 0 only, as ``finish`` adds the groups).
    static __device__ __forceinline__ void load_state(Acc& a, int g, size_t qi, const AttnParams& p) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) a.o[db] = *reinterpret_cast<const f32x4*>(p.st_o + qi * D + db * 16 + 4 * g);
        a.m = p.st_m[qi];
        a.l = g == 0 ? p.st_l[qi] : 0.f;
        if constexpr (SEARCH) {
            a.bc = p.st_bc[qi];
            a.bs = p.st_bs[qi];
        }
    }

    static __device__ __forceinline__ Src src_of(const AttnParams& p, int h) {
        Src s;
        s.ka = static_cast<const T*>(p.ka) + static_cast<size_t>(h) * p.a_rows * D;
        s.va = HAS_V ? static_cast<const T*>(p.va) + static_cast<size_t>(h) * p.a_rows * D : nullptr;
        s.kb = p.kb ? static_cast<const T*>(p.kb) + static_cast<size_t>(h) * p.b_rows * D : nullptr;
        s.vb = (HAS_V && p.vb) ? static_cast<const T*>(p.vb) + static_cast<size_t>(h) * p.b_rows * D : nullptr;
        s.kn = SEARCH ? p.knorm + static_cast<size_t>(h) * p.a_rows : nullptr;
        s.kcnt = BIAS ? p.kcount + static_cast<size_t>(h) * p.a_rows : nullptr;
        s.ida = MULTI && p.ida ? p.ida + static_cast<size_t>(h) * p.a_rows : nullptr;
        s.idb = MULTI && p.idb ? p.idb + static_cast<size_t>(h) * p.b_rows : nullptr;
        s.na = 0;
        return s;
    }
};

// AnnCA prompt selection done by the attention block itself (FAST-AR blog,
// "2. AnnCA"; summary, "2. Core Components" B): the buckets occupied by
// frame f's queries form a bitmap in LDS, and the prompt tokens whose bucket
// bit is set become the block's key list in ascending order, written straight
// into ``kidx``; the rest of the last tile holds row 0 (any valid row: those
// scores are masked).  Every block of the frame builds the same list (the ids
// are a few KB, read through L2); the frame's first block also writes the
// keep mask and count.  Needs L <= KCH, so the list is a single staged chunk.
// Returns the number of kept tokens.
// AnnCA block coordinates (head h, frame f, query block c) from the block id.
// The chip hands blocks to its eight XCDs in turn by linear id, and each XCD
// has its own L2.  The id is re-mapped (a bijection on [0, blocks)) so that
// consecutive logical blocks -- the query blocks of one (head, frame), which
// all gather the same selected prompt rows -- run on one XCD and re-read
// those rows from its L2.
__device__ __forceinline__ void ca_block_coords(int& h, int& f, int& c) {
    const int gx = gridDim.x, gy = gridDim.y;
    const int b = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
#if CA_XCD
    constexpr int X = 8;
    const int nb = gx * gy * gridDim.z;
    const int per = nb / X, rem = nb % X, x = b % X;
    const int l = x * per + min(x, rem) + b / X;
#else
    const int l = b;
#endif
    c = __builtin_amdgcn_readfirstlane(l % gx);             // uniform: scalar registers
    f = __builtin_amdgcn_readfirstlane((l / gx) % gy);
    h = __builtin_amdgcn_readfirstlane(l / (gx * gy));
}

// AnnSA / TOP1 block coordinates (head h, work item) from the block id of a
// (heads, max_items) grid.  Blocks go to the eight XCDs in turn by linear id,
// each XCD with its own L2; a bucket whose queries fill several items has
// those items next to one another in its head's list, and they gather the
// same key rows.  So runs of SA_XCD_RUN consecutive items of one head are
// dealt to one XCD, where they run one after another and the later ones find
// the rows in that L2.  Runs are dealt to the XCDs in turn, in the list's
// order (heads fastest, longest items first); the blocks past the last full
// round of eight runs (the end of every list: short items and padding) keep
// the plain order.  A bijection on the grid: max_items is a multiple of 8.
static_assert(SA_XCD_RUN >= 1 && 8 % SA_XCD_RUN == 0, "runs must divide the item count's multiple of 8");
__device__ __forceinline__ void sa_block_coords(int& h, int& item) {
    const int H = gridDim.x, M = gridDim.y;
    const int b = blockIdx.x + H * blockIdx.y;
    constexpr int G = SA_XCD_RUN, X = 8;
    const int full = (H * M / G / X) * X * G;    // blocks in full rounds
    int l = b;
    if (b < full) {
        const int s = b / X;
        l = ((s / G) * X + b % X) * G + s % G;
    }
    const int run = l / G;
    // uniform values out of a vector division: back to scalar registers, so
    // the head's row pointers stay scalar too
    h = __builtin_amdgcn_readfirstlane(run % H);
    item = __builtin_amdgcn_readfirstlane((run / H) * G + l % G);
}

// AnnCA prompt selection inside the attention block (prompts of up to
// kCaFusedMaxL tokens): a prompt token is kept when some query of the frame
// falls in its bucket (FAST-AR blog, "2. AnnCA").  In two parts, so that the
// id loads are issued ahead of the query rows and do not queue behind them:
// ca_select_issue loads the prompt ids (clamped indices, no branch) and the
// frame's query ids (16-byte loads of 8 ids; the at most 7 ids before and
// after the aligned part one per thread); ca_select_finish marks each
// query's bucket in a byte-per-bucket LDS table, then one block scan over the
// threads' kept counts writes the kept prompt positions, in ascending order,
// to kidx (padded with 0 to a whole key tile).
template <int NT>
struct CaSel {
    static constexpr int PU = KCH / NT;          // consecutive prompt tokens per thread
    uint32_t pid[PU];
    uint32_t id_pre, id_tail;
    u32x4 r[4];
    const u32x4* qv;
    const uint16_t* qi;
    int n, pre, nv, tail;
};

template <int NT>
__device__ __forceinline__ void ca_select_issue(const AttnParams& p, int h, int f, CaSel<NT>& S) {
    static_assert(kCaFusedMaxL == KCH, "the kept list fills at most one index chunk");
    const int tid = threadIdx.x, L = p.L;
    const uint16_t* pi = p.ca_kp_ids + static_cast<size_t>(h) * L;
    if (L > 0) {
#pragma unroll
        for (int u = 0; u < CaSel<NT>::PU; ++u) S.pid[u] = pi[min(tid * CaSel<NT>::PU + u, L - 1)];
    }
    S.qi = p.q_ids + static_cast<size_t>(h) * p.Nq + static_cast<size_t>(f) * p.frame_len;
    S.n = p.frame_len;
    S.pre = min(S.n, static_cast<int>(((16u - (reinterpret_cast<uintptr_t>(S.qi) & 15u)) & 15u) >> 1));
    S.nv = (S.n - S.pre) >> 3;
    S.tail = S.pre + S.nv * 8;
    S.qv = reinterpret_cast<const u32x4*>(S.qi + S.pre);
    S.id_pre = S.qi[min(tid, S.n - 1)];
    S.id_tail = S.qi[min(S.tail + tid, S.n - 1)];
    if (S.nv > 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) S.r[u] = S.qv[min(u * NT + tid, S.nv - 1)];
    }
}

template <int NT>
__device__ __forceinline__ int ca_select_finish(const AttnParams& p, int h, int f, int* kidx, bool first,
                                                CaSel<NT>& S) {
    constexpr int PU = CaSel<NT>::PU;
    __shared__ __align__(16) uint8_t flag[kCaMaxBuckets];
    __shared__ int sscan[NT / kWave];
    const int tid = threadIdx.x, L = p.L;
    const uint32_t mask = static_cast<uint32_t>(p.ca_buckets - 1);
    const size_t row = static_cast<size_t>(h) * p.F + f;
    // Every query of a bucket stores the same 1, so the stores need no
    // atomics (many queries share a bucket: atomics on a bitmap word would
    // serialise them).
    auto mark_all = [&](int v0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (v0 + u * NT + tid < S.nv) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    flag[S.r[u][e] & mask] = 1;
                    flag[(S.r[u][e] >> 16) & mask] = 1;
                }
            }
        }
    };
    for (int i = tid; i < (p.ca_buckets + 3) / 4; i += NT) reinterpret_cast<uint32_t*>(flag)[i] = 0;
    __syncthreads();
    if (S.nv > 0) mark_all(0);
    for (int v0 = 4 * NT; v0 < S.nv; v0 += 4 * NT) {
#pragma unroll
        for (int u = 0; u < 4; ++u) S.r[u] = S.qv[min(v0 + u * NT + tid, S.nv - 1)];
        mark_all(v0);
    }
    if (tid < S.pre) flag[S.id_pre & mask] = 1;
    if (tid < S.n - S.tail) flag[S.id_tail & mask] = 1;
    __syncthreads();
    int keep[PU], cnt = 0;
#pragma unroll
    for (int u = 0; u < PU; ++u) {
        keep[u] = tid * PU + u < L ? static_cast<int>(flag[S.pid[u] & mask]) : 0;
        cnt += keep[u];
    }
    int total;
    int pos = block_exclusive_scan<NT>(cnt, sscan, total);
#pragma unroll
    for (int u = 0; u < PU; ++u) {
        const int t = tid * PU + u;
        if (keep[u]) kidx[pos++] = t;
        if (first && p.ca_keep && t < L) p.ca_keep[row * L + t] = static_cast<uint8_t>(keep[u]);
    }
    const int end = (total + KT - 1) / KT * KT;
    for (int i = total + tid; i < end; i += NT) kidx[i] = 0;
    if (first && p.ca_keep_count && tid == 0) p.ca_keep_count[row] = total;
    __syncthreads();
    return total;
}

}  // namespace

// NW waves per block; the item is 16*NW queries (SA / TOP1: the 64-query
// slices of the bucket sort, NW = 4).
template <typename T, int D, int MODE, bool SEARCH, typename OT, int NW, bool BIAS = false,
          bool MULTI = false>
__device__ __forceinline__ void attn_body(const AttnParams& p) {
    constexpr int NT = 64 * NW, QT = 16 * NW;
    static_assert(MODE == MODE_CA || QT == kQTile, "SA / TOP1 items are kQTile queries");
    using B = Blk<T, D, MODE, SEARCH, NT, BIAS, MULTI>;
    __shared__ __align__(16) T Ks[KT * B::STRK];
    __shared__ __align__(16) T Vs[B::HAS_V ? KT * B::STRV : 1];
    __shared__ __align__(16) int kslot[SEARCH ? KT : 4];
    __shared__ __align__(16) float kinv[SEARCH ? KT : 4];
    __shared__ __align__(16) float kbias[BIAS ? KT : 4];
    __shared__ __align__(16) int kid[MULTI ? KT : 4];
    __shared__ int sslot[2][B::SLOTS ? KT : 1];
    __shared__ int kidx[KCH];
    const typename B::Smem sm{Ks, Vs, kslot, kinv, kbias, kid};
    const float inv_c = BIAS ? 1.f / p.scale_log2 : 0.f;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;

    int h, q_count, nk, qbase = 0;
    const int32_t* qlist = nullptr;
    const int32_t* klist;
    // AnnCA blocks that select their prompt keys themselves hold the whole
    // key list in ``kidx`` from here on
    const bool fused = MODE == MODE_CA && p.ca_fused != 0;
    if constexpr (MODE == MODE_CA) {
        int f, c;
        ca_block_coords(h, f, c);
        qbase = f * p.frame_len + c * QT;
        q_count = min(QT, p.frame_len - c * QT);
        if (fused) {
            CaSel<NT> S;
            ca_select_issue<NT>(p, h, f, S);
            nk = ca_select_finish<NT>(p, h, f, kidx, c == 0, S);
            klist = nullptr;
        } else {
            nk = p.ca_cnt[h * p.F + f];
            klist = p.ca_idx + (static_cast<size_t>(h) * p.F + f) * p.L;
        }
    } else {
        int item;
        sa_block_coords(h, item);               // heads fastest: the longest items of every head first
        const int4 it = p.items[static_cast<size_t>(h) * p.max_items + item];
        if (it.y <= 0) return;
        q_count = it.y;
        qlist = p.qperm + static_cast<size_t>(h) * p.qperm_stride + it.x;
        nk = it.w;
        klist = p.kperm + static_cast<size_t>(h) * p.kperm_stride + it.z;
    }
    typename B::Src sr = B::src_of(p, h);
    if constexpr (MODE == MODE_SA) sr.na = clamp_n(p.n_valid, h, p.cap);

    const int ql = w * 16 + c16;
    const bool qvalid = ql < q_count;
    const bool wave_active = w * 16 < q_count;

    // The key list is staged in LDS (KCH entries at a time, coalesced), so the
    // gathers never wait on a dependent index load.  Entries past the end
    // repeat the last key, so every lane of a partial tile still gathers a
    // valid row (its score is masked).  The first chunk is loaded before the
    // query rows' indices, so the two index loads are in flight together and
    // the first K/V gathers start while the query rows are still on their way.
    auto stage_idx = [&](int first) __attribute__((always_inline)) {
        for (int i = tid; i < KCH; i += NT) {
            const int r = first + i;
            kidx[i] = nk > 0 ? klist[r < nk ? r : nk - 1] : 0;
        }
    };
    static_assert(KCH % NT == 0, "key chunk split");
    int kfirst[KCH / NT];
    if (!fused) {
#pragma unroll
        for (int u = 0; u < KCH / NT; ++u) {
            const int r = tid + u * NT;
            kfirst[u] = nk > 0 ? klist[r < nk ? r : nk - 1] : 0;
        }
    }
    int qrow = 0;
    if (qvalid) qrow = (MODE == MODE_CA) ? qbase + ql : qlist[ql];
    const T* qh = static_cast<const T*>(p.q) + static_cast<size_t>(h) * p.Nq * D;

    typename B::QF qf;
    B::load_q(qf, qvalid ? qh + static_cast<size_t>(qrow) * D : nullptr, g);

    typename B::Acc acc;
    acc.reset();
    const size_t qi = static_cast<size_t>(h) * p.Nq + qrow;
    typename B::Seen seen{0, 0, 0};
    if constexpr (MULTI) {
        seen = typename B::Seen{qvalid ? static_cast<int>(p.q_ids[qi]) : 0, p.table, p.fbits};
        if (p.table > 0 && qvalid) B::load_state(acc, g, qi, p);
    }
    const int nt = (nk + KT - 1) / KT;

    // One pipeline step on tile t: store its K (stage S) and V (stage VS),
    // refill VS with V of tile t+1 and S with K of tile t+2, compute on tile
    // t.  K runs two tiles ahead, V one: three tiles' rows in registers
    // instead of four, so three waves fit on a SIMD.  The V indices of tile
    // t+1 are read before a new index chunk may overwrite them (the barrier
    // before the chunk's staging keeps every wave's reads ahead of it).
    typename B::Stage VS;
    auto step = [&](typename B::Stage& S, int t) __attribute__((always_inline)) {
        if (t >= nt) return;                              // block-uniform
        __syncthreads();
        B::store_tile(S, sm, sr.na, tid, inv_c, &VS);
        __syncthreads();
        if (t + 1 < nt) B::template load_tile<false, true>(VS, kidx, t + 1, sr, tid);
        if (t + 2 < nt) {
            if (((t + 2) * KT) % KCH == 0) {        // next index chunk
                __syncthreads();
                stage_idx((t + 2) * KT);
                __syncthreads();
            }
            B::template load_tile<true, false>(S, kidx, t + 2, sr, tid);
        }
        if (wave_active) B::compute_tile(acc, qf, sm, t * KT, nk, sr.na, p.scale_log2, g, c16, seen);
    };

    typename B::Stage A, Bs;
    A.slots = sslot[0];
    Bs.slots = sslot[1];
    VS.slots = nullptr;
    if (!fused) {
#pragma unroll
        for (int u = 0; u < KCH / NT; ++u) kidx[tid + u * NT] = kfirst[u];
    }
    __syncthreads();
    if (nt > 0) {
        B::template load_tile<true, false>(A, kidx, 0, sr, tid);
        B::template load_tile<false, true>(VS, kidx, 0, sr, tid);
    }
    if (nt > 1) B::template load_tile<true, false>(Bs, kidx, 1, sr, tid);
    // Each stage is named in exactly one place of a fixed pair of steps, so
    // both keep fixed registers.  A step past the last tile does nothing.
#pragma unroll 1
    for (int t = 0; t < nt; t += 2) {
        step(A, t);
        step(Bs, t + 1);
    }

    if (MULTI && p.table + 1 < p.tables) {
        B::store_state(acc, qvalid, g, qi, p);
        return;
    }
    B::finish_q(qf);                          // 1/|q|, needed by the search's cosine only
    B::template finish<OT>(acc, qf, qvalid, g, static_cast<OT*>(p.out) + qi * D, p.lse ? p.lse + qi : nullptr,
                           p.best ? p.best + qi : nullptr, p.bcos ? p.bcos + qi : nullptr, p.scale_log2);
}

// Two 16-query groups per wave (32 queries per wave, 32*NW per block): the
// same gather pipeline as attn_body, with every K/V fragment read from LDS
// used by both groups.  MODE_CA: AnnCA, one block per (head, frame, 32*NW
// consecutive queries).  MODE_SA: AnnSA over items of kQTileWide queries (the
// bucket sort's slices when buckets average that many queries), for large
// buckets: each gathered K/V tile then serves four times the queries of a
// 64-query item, so the head's keys are re-read a quarter as often.  No
// search, group-size shift or tables in this form.
template <typename T, int D, int MODE, typename OT, int NW, int NG>
__device__ __forceinline__ void attn_wide_body(const AttnParams& p) {
    constexpr int NT = 64 * NW, QT = 16 * NG * NW;
    static_assert(MODE == MODE_CA || QT == kQTileWide, "wide AnnSA items are kQTileWide queries");
    using B = Blk<T, D, MODE, false, NT>;
    __shared__ __align__(16) T Ks[KT * B::STRK];
    __shared__ __align__(16) T Vs[KT * B::STRV];
    __shared__ int sslot[2][1];
    __shared__ int kidx[KCH];
    const typename B::Smem sm{Ks, Vs, nullptr, nullptr, nullptr, nullptr};

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    int h, q_count, nk, qbase = 0, ca_f = 0, ca_c = 0;
    const int32_t* qlist = nullptr;
    const int32_t* klist;
    // as in attn_body; here the selection's id loads are issued first, then
    // the query rows, and the selection runs while the rows are on their way
    const bool fused = MODE == MODE_CA && p.ca_fused != 0;
    if constexpr (MODE == MODE_CA) {
        ca_block_coords(h, ca_f, ca_c);
        const int f = ca_f, c = ca_c;
        qbase = f * p.frame_len + c * QT;
        q_count = min(QT, p.frame_len - c * QT);
        if (fused) {
            nk = 0;
            klist = nullptr;
        } else {
            nk = p.ca_cnt[h * p.F + f];
            klist = p.ca_idx + (static_cast<size_t>(h) * p.F + f) * p.L;
        }
    } else {
        int item;
        sa_block_coords(h, item);               // as in attn_body
        const int4 it = p.items[static_cast<size_t>(h) * p.max_items + item];
        if (it.y <= 0) return;
        q_count = it.y;
        qlist = p.qperm + static_cast<size_t>(h) * p.qperm_stride + it.x;
        nk = it.w;
        klist = p.kperm + static_cast<size_t>(h) * p.kperm_stride + it.z;
    }
    typename B::Src sr = B::src_of(p, h);
    if constexpr (MODE == MODE_SA) sr.na = clamp_n(p.n_valid, h, p.cap);

    // the first chunk of the key list is loaded before the query rows, so the
    // first K/V gathers need not wait for them
    static_assert(KCH % NT == 0, "key chunk split");
    int kfirst[KCH / NT];
    if (!fused) {
#pragma unroll
        for (int u = 0; u < KCH / NT; ++u) {
            const int r = tid + u * NT;
            kfirst[u] = nk > 0 ? klist[r < nk ? r : nk - 1] : 0;
        }
    }
    CaSel<NT> csel;
    if (fused) ca_select_issue<NT>(p, h, ca_f, csel);
    const T* qh = static_cast<const T*>(p.q) + static_cast<size_t>(h) * p.Nq * D;
    typename B::QF qf[NG];
    typename B::Acc acc[NG];
    bool qvalid[NG];
    int qrow[NG];
#pragma unroll
    for (int qg = 0; qg < NG; ++qg) {
        const int ql = w * 16 * NG + qg * 16 + c16;
        qvalid[qg] = ql < q_count;
        if constexpr (MODE == MODE_CA) {
            // a query past the frame's end reads the frame's first row (its
            // output is never written), so the row loads carry no branch
            qrow[qg] = qbase + (qvalid[qg] ? ql : 0);
            B::load_q_row(qf[qg], qh + static_cast<size_t>(qrow[qg]) * D, g);
        } else {
            qrow[qg] = qvalid[qg] ? qlist[ql] : 0;
            B::load_q(qf[qg], qvalid[qg] ? qh + static_cast<size_t>(qrow[qg]) * D : nullptr, g);
        }
        acc[qg].reset();
    }
    const bool wave_active = w * 16 * NG < q_count;
    if (fused) nk = ca_select_finish<NT>(p, h, ca_f, kidx, ca_c == 0, csel);

    auto stage_idx = [&](int first) __attribute__((always_inline)) {
        for (int i = tid; i < KCH; i += NT) {
            const int r = first + i;
            kidx[i] = nk > 0 ? klist[r < nk ? r : nk - 1] : 0;
        }
    };
    const int nt = (nk + KT - 1) / KT;
    auto step = [&](typename B::Stage& S, int t) __attribute__((always_inline)) {
        if (t >= nt) return;                              // block-uniform
        __syncthreads();
        B::store_tile(S, sm, sr.na, tid, 0.f);
        __syncthreads();
        if (t + 2 < nt) {
            if (((t + 2) * KT) % KCH == 0) {
                stage_idx((t + 2) * KT);
                __syncthreads();
            }
            B::load_tile(S, kidx, t + 2, sr, tid);
        }
        if (wave_active) B::template compute_tileg<NG>(acc, qf, sm, t * KT, nk, p.scale_log2, g, c16);
    };
    typename B::Stage A, Bs;
    A.slots = sslot[0];
    Bs.slots = sslot[1];
    if (!fused) {
#pragma unroll
        for (int u = 0; u < KCH / NT; ++u) kidx[tid + u * NT] = kfirst[u];
    }
    __syncthreads();
    if (nt > 0) B::load_tile(A, kidx, 0, sr, tid);
    if (nt > 1) B::load_tile(Bs, kidx, 1, sr, tid);
#pragma unroll 1
    for (int t = 0; t < nt; t += 2) {
        step(A, t);
        step(Bs, t + 1);
    }
#pragma unroll
    for (int qg = 0; qg < NG; ++qg) {
        const size_t qi = static_cast<size_t>(h) * p.Nq + qrow[qg];
        B::template finish<OT>(acc[qg], qf[qg], qvalid[qg], g, static_cast<OT*>(p.out) + qi * D,
                               (MODE == MODE_SA && p.lse) ? p.lse + qi : nullptr, nullptr, nullptr,
                               p.scale_log2);
    }
}

// NG query groups per wave: two at two waves per SIMD; four at one (their
// accumulators need the whole register file).
template <typename T, int D, int MODE, typename OT, int NW, int NG = 2>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NG >= 4 ? 1 : 2, NG >= 4 ? 1 : 2)))
void attn_wide_kernel(const AttnParams p) {
    attn_wide_body<T, D, MODE, OT, NW, NG>(p);
}

// K+V modes keep two prefetched tiles of K and V in registers: up to 256
// registers per lane, i.e. 2 waves per SIMD.
#ifndef KV_WAVES
#define KV_WAVES 3
#endif
template <typename T, bool BIAS, bool MULTI>
constexpr int kv_waves() { return (sizeof(T) == 2 && !BIAS && !MULTI) ? KV_WAVES : 2; }
template <typename T, int D, int MODE, bool SEARCH, typename OT, int NW, bool BIAS = false,
          bool MULTI = false>
__global__ __launch_bounds__(64 * NW)
__attribute__((amdgpu_waves_per_eu(kv_waves<T, BIAS, MULTI>(), kv_waves<T, BIAS, MULTI>())))
void attn_kv_kernel(const AttnParams p) {
    attn_body<T, D, MODE, SEARCH, OT, NW, BIAS, MULTI>(p);
}

// The search alone stages K only and runs at the occupancy its registers allow.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_top1_kernel(const AttnParams p) {
    attn_body<T, D, MODE_TOP1, true, float, 4>(p);
}

namespace {

// AnnCA blocks take 16*kCaGroups*kCaWaves consecutive queries of a frame
// (16*kCaWaves where a wave keeps one group): every K/V tile gathered into
// LDS serves that many queries.  Blocks of 128 queries: the 256-query form
// is faster alone (31.6 vs 33.5 us at the Wan-1.3B chunk) but slower in the
// step, where AnnCA shares the CUs with the commit's kernels.
constexpr int kCaWaves = CA_WAVES;
constexpr int kCaGroups = CA_GROUPS;
template <typename T, int D>
constexpr bool ca_grouped() { return kCaGroups >= 2 && (sizeof(T) == 2 || D == 64); }
template <typename T, int D>
constexpr int ca_block_queries() { return 16 * (ca_grouped<T, D>() ? kCaGroups : 1) * kCaWaves; }

template <typename T, int D, int MODE, typename OT>
void attn_go(int H, const AttnParams& p, hipStream_t s) {
    dim3 grid;
    if constexpr (MODE == MODE_CA) {
        constexpr int QB = ca_block_queries<T, D>();
        grid = dim3((p.frame_len + QB - 1) / QB, p.F, H);
    } else {
        grid = dim3(H, p.max_items);
    }
    if (grid.x == 0 || grid.y == 0 || grid.z == 0) return;
    if constexpr (MODE == MODE_TOP1) {
        hipLaunchKernelGGL((attn_top1_kernel<T, D>), grid, dim3(256), 0, s, p);
    } else if constexpr (MODE == MODE_SA) {
        const bool bias = p.kcount != nullptr && p.a_rows > 0;
        const bool search = p.best != nullptr;
#define FASTAR_SA(S_, B_, M_) \
    hipLaunchKernelGGL((attn_kv_kernel<T, D, MODE_SA, S_, OT, 4, B_, M_>), grid, dim3(256), 0, s, p)
        if constexpr (sizeof(T) == 2 || D == 64) {
            if (p.wide) {
                // the host asks for it only without search, group sizes or tables
                hipLaunchKernelGGL((attn_wide_kernel<T, D, MODE_SA, OT, kQTileWide / 32>), grid,
                                   dim3(2 * kQTileWide), 0, s, p);
                return;
            }
        }
        if (p.tables > 1) {
            if (search) { if (bias) FASTAR_SA(true, true, true); else FASTAR_SA(true, false, true); }
            else { if (bias) FASTAR_SA(false, true, true); else FASTAR_SA(false, false, true); }
        } else {
            if (search) { if (bias) FASTAR_SA(true, true, false); else FASTAR_SA(true, false, false); }
            else { if (bias) FASTAR_SA(false, true, false); else FASTAR_SA(false, false, false); }
        }
#undef FASTAR_SA
    } else if constexpr (ca_grouped<T, D>()) {
        // (fp32 with d = 128 keeps one group per wave: two would spill)
        hipLaunchKernelGGL((attn_wide_kernel<T, D, MODE_CA, OT, kCaWaves, kCaGroups>), grid, dim3(64 * kCaWaves),
                           0, s, p);
    } else {
        hipLaunchKernelGGL((attn_kv_kernel<T, D, MODE_CA, false, OT, kCaWaves>), grid, dim3(64 * kCaWaves), 0,
                           s, p);
    }
}

template <int MODE>
void attn_dispatch(bool bf16, int d, bool out_bf16, int H, const AttnParams& p, hipStream_t s) {
    if (bf16) {
        if (d == 64) {
            out_bf16 ? attn_go<uint16_t, 64, MODE, uint16_t>(H, p, s) : attn_go<uint16_t, 64, MODE, float>(H, p, s);
        } else {
            out_bf16 ? attn_go<uint16_t, 128, MODE, uint16_t>(H, p, s) : attn_go<uint16_t, 128, MODE, float>(H, p, s);
        }
    } else {
        if (d == 64) {
            out_bf16 ? attn_go<float, 64, MODE, uint16_t>(H, p, s) : attn_go<float, 64, MODE, float>(H, p, s);
        } else {
            out_bf16 ? attn_go<float, 128, MODE, uint16_t>(H, p, s) : attn_go<float, 128, MODE, float>(H, p, s);
        }
    }
}

}  // namespace

hipError_t launch_attn(int mode, bool bf16, int d, bool out_bf16, int H, const AttnParams& params,
                       hipStream_t s) {
    if (H == 0) return hipSuccess;
    AttnParams p = params;
    p.H = H;
    switch (mode) {
        case MODE_SA:
            timer_begin("annsa_attn", s);
            attn_dispatch<MODE_SA>(bf16, d, out_bf16, H, p, s);
            break;
        case MODE_CA:
            timer_begin("annca_attn", s);
            attn_dispatch<MODE_CA>(bf16, d, out_bf16, H, p, s);
            break;
        default:
            timer_begin("tempcache_top1", s);
            attn_dispatch<MODE_TOP1>(bf16, d, false, H, p, s);
            break;
    }
    timer_end(s);
    return hipGetLastError();
}

}  // namespace fastar
