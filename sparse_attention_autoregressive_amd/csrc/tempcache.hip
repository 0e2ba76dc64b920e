// TempCache commit (FAST-AR blog, "1. TempCache"; summary, "2. Core
// Components" A).  Given each current token's top-1 (best slot, cosine), one
// block per head
//   1. resets the claim entries of the slots this chunk matched and lets every
//      matched token claim its slot with atomicMax of its index, so the most
//      recent token wins regardless of scheduling,
//   2. resolves the matched tokens (winner -> its slot, marked in a bitmap of
//      refreshed slots; others dropped), counts the winners and ranks the
//      unmatched tokens in token order with one block scan (ranks stay in
//      registers when the chunk fits one pass of the block),
//   3. if the cache overflows, selects the e non-refreshed slots with the
//      smallest (timestamp, slot) by a radix select on the timestamps
//      (8-bit digits of ts - min(ts); one pass when timestamps span < 256)
//      and lists them in slot order (two block scans); the search runs over
//      the N oldest slots when an order kernel has listed them beforehand
//      (they always hold the answer, see tc_order_kernel), else over every
//      slot, 32 consecutive slots (one bitmap word) per thread,
//   4. writes the unmatched tokens' destinations, the eviction list, the counts
//      and the new valid-slot count;
// then a copy kernel moves the written tokens' rows into place (16 lanes per
// token) and records each written key's norm.  Every decision
// is integer or a single fp32 compare, so results are deterministic.
//
// Mean-merged caches (summary, "2. Core Components" A, Lemma 5.1: a slot
// holds the mean value of a group of tokens with one key) use the same
// decisions.  The select also groups the matched tokens by the token that
// represents their slot (group sizes by integer atomics, offsets by a block
// scan, members placed at atomic positions), and the merge scatter, one wave
// per written token, folds a group's values into its slot in ascending token
// order -- the members are ordered in registers first, so the fp32 sum, and
// the cache, do not depend on the order the atomics ran in.
#include "common.hpp"
#include "launch.hpp"

namespace fastar {

namespace {
constexpr int SEL_NT = 1024;
constexpr int TOK_ITEMS = 8;                      // tokens per thread per chunk
constexpr int TOK_CHUNK = SEL_NT * TOK_ITEMS;     // < 65536: packed counters fit 16 bits
constexpr int SLOT_ITEMS = 32;                    // slots per thread per chunk (one bitmap word)
constexpr int SLOT_CHUNK = SEL_NT * SLOT_ITEMS;
// Caches up to this many slots keep the select's claim table and refreshed
// bitmap in LDS (4 bytes + 1 bit per slot: 132 KiB at the limit).
constexpr int kLdsClaimSlots = 32768;
// Dynamic LDS the select may take (the 160 KiB of a workgroup less room for
// its static arrays, about 1.2 KiB).
constexpr size_t kSelectDynLds = 160 * 1024 - 2048;

__device__ __forceinline__ uint32_t ts_key(int32_t t) { return static_cast<uint32_t>(t) ^ 0x80000000u; }

// Block-wide min and max of one value per thread, reduced together.
__device__ __forceinline__ void block_min_max(uint32_t& mn, uint32_t& mx, uint32_t* red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const uint32_t a = __shfl_xor(mn, off), b = __shfl_xor(mx, off);
        mn = a < mn ? a : mn;
        mx = b > mx ? b : mx;
    }
    const int w = threadIdx.x / kWave;
    if (lane_id() == 0) {
        red[2 * w] = mn;
        red[2 * w + 1] = mx;
    }
    __syncthreads();
    mn = red[0];
    mx = red[1];
    for (int i = 1; i < SEL_NT / kWave; ++i) {
        mn = red[2 * i] < mn ? red[2 * i] : mn;
        mx = red[2 * i + 1] > mx ? red[2 * i + 1] : mx;
    }
    __syncthreads();
}

__device__ __forceinline__ bool is_matched(int b, float c, int n, float tau) {
    return b >= 0 && b < n && c >= tau;
}
}  // namespace

// ------------------------------------------------------------ eviction search
// Sources of the eviction search: a sequence of positions, ITEMS consecutive
// ones per thread, each standing for a cache slot with a key (its timestamp,
// order-preserving as unsigned) and a candidate bit.
namespace {
// Every slot 0..n-1, 32 per thread (one refreshed-bitmap word).  refr null:
// every valid slot is a candidate.
struct SlotRange {
    static constexpr int ITEMS = SLOT_ITEMS;
    const int32_t* ts;
    const uint32_t* refr;
    int n;
    uint32_t key[ITEMS];
    uint32_t cand = 0;
    int base = 0, cached = -1;
    __device__ SlotRange(const int32_t* t, const uint32_t* r, int n_) : ts(t), refr(r), n(n_) {}
    __device__ __forceinline__ void load(int c0) {
        if (cached == c0) return;
        cached = c0;
        base = c0 + static_cast<int>(threadIdx.x) * ITEMS;
        const bool vec = base + ITEMS <= n && (reinterpret_cast<uintptr_t>(ts + base) & 15) == 0;
        if (vec) {
#pragma unroll
            for (int k = 0; k < ITEMS; k += 4) {
                const int4 t = *reinterpret_cast<const int4*>(ts + base + k);
                key[k] = ts_key(t.x); key[k + 1] = ts_key(t.y);
                key[k + 2] = ts_key(t.z); key[k + 3] = ts_key(t.w);
            }
        } else {
            // clamped indices, no branch (n >= 1 when called)
#pragma unroll
            for (int k = 0; k < ITEMS; ++k) key[k] = ts_key(ts[min(base + k, n - 1)]);
#pragma unroll
            for (int k = 0; k < ITEMS; ++k)
                if (base + k >= n) key[k] = 0u;
        }
        const int left = n - base;
        const uint32_t valid = left >= ITEMS ? 0xFFFFFFFFu : (left > 0 ? (1u << left) - 1u : 0u);
        if (refr) {                                     // uniform
            const uint32_t rw = refr[min(base, n - 1) >> 5];           // no branch on the load
            cand = ~rw & valid;
        } else {
            cand = valid;
        }
    }
    __device__ __forceinline__ int slot(int k) const { return base + k; }
};

// The slots of a list (ascending), 8 per thread; entries outside [0, n) are
// no candidates (a list from another cache state gives wrong evictions, never
// an access outside the cache).
struct SlotList {
    static constexpr int ITEMS = 8;
    const int32_t* list;
    const int32_t* ts;
    const uint32_t* refr;
    int m, n;
    uint32_t key[ITEMS];
    int sl[ITEMS];
    uint32_t cand = 0;
    int cached = -1;
    __device__ SlotList(const int32_t* l, const int32_t* t, const uint32_t* r, int m_, int n_)
        : list(l), ts(t), refr(r), m(m_), n(n_) {}
    __device__ __forceinline__ void load(int c0) {
        if (cached == c0) return;
        cached = c0;
        const int base = c0 + static_cast<int>(threadIdx.x) * ITEMS;
        // clamped indices, no branch: all loads in flight at once (m >= 1)
#pragma unroll
        for (int k = 0; k < ITEMS; ++k) sl[k] = list[min(base + k, m - 1)];
#pragma unroll
        for (int k = 0; k < ITEMS; ++k)
            if (base + k >= m) sl[k] = -1;
        cand = 0;
#pragma unroll
        for (int k = 0; k < ITEMS; ++k) {
            const bool in = static_cast<unsigned>(sl[k]) < static_cast<unsigned>(n);
            if (!in) sl[k] = 0;
            key[k] = ts_key(ts[sl[k]]);
            if (in && !((refr[sl[k] >> 5] >> (sl[k] & 31)) & 1u)) cand |= 1u << k;
        }
    }
    __device__ __forceinline__ int slot(int k) const { return sl[k]; }
};
}  // namespace

// The e candidates of smallest (key, position) among positions 0..n_items-1
// of ``src``, written to out[0..e) in position order (as slots).  A radix
// select on 8-bit digits of key - min(key) (one pass when the keys span
// < 256) finds the e-th key tstar and how many of the candidates equal to it
// are taken; one packed block scan then gives every thread the list position
// of its first selected item.  Needs at least e candidates; block-wide (every
// thread of the SEL_NT-thread block calls it).
template <class Src>
__device__ __forceinline__ void select_smallest(Src& src, int n_items, int e, int32_t* out, int* smem,
                                                uint32_t* red, int* hist, int* bcast) {
    constexpr int ITEMS = Src::ITEMS;
    constexpr int CHUNK = SEL_NT * ITEMS;
    const int tid = threadIdx.x;
    uint32_t lmin = 0xFFFFFFFFu, lmax = 0u;
    for (int c0 = 0; c0 < n_items; c0 += CHUNK) {
        src.load(c0);
#pragma unroll
        for (int k = 0; k < ITEMS; ++k)
            if ((src.cand >> k) & 1) {
                lmin = src.key[k] < lmin ? src.key[k] : lmin;
                lmax = src.key[k] > lmax ? src.key[k] : lmax;
            }
    }
    uint32_t kmin = lmin, kmax = lmax;
    block_min_max(kmin, kmax, red);
    uint32_t prefix = 0;
    int need = e;
    if (kmax != kmin) {
        const uint32_t range = kmax - kmin;
        const int nbits = 32 - __clz(static_cast<int>(range));
        for (int shift = ((nbits - 1) / 8) * 8; shift >= 0; shift -= 8) {
            if (tid < 256) hist[tid] = 0;
            __syncthreads();
            for (int c0 = 0; c0 < n_items; c0 += CHUNK) {
                src.load(c0);
                // neighbouring items usually share a timestamp: add runs of
                // equal digits with one atomic each
                int rd = -1, rc = 0;
#pragma unroll
                for (int k = 0; k < ITEMS; ++k) {
                    if ((src.cand >> k) & 1) {
                        const uint32_t rel = src.key[k] - kmin;
                        const uint32_t hi = (shift + 8 >= 32) ? 0u : (rel >> (shift + 8));
                        if (hi == prefix) {
                            const int dg = static_cast<int>((rel >> shift) & 255u);
                            if (dg != rd) {
                                if (rc) atomicAdd(&hist[rd], rc);
                                rd = dg;
                                rc = 0;
                            }
                            ++rc;
                        }
                    }
                }
                if (rc) atomicAdd(&hist[rd], rc);
            }
            __syncthreads();
            // the digit holding the need-th candidate: a scan over the 256
            // bins, owned by the one thread whose bin straddles it
            const int v = tid < 256 ? hist[tid] : 0;
            int tot;
            const int ex = block_exclusive_scan<SEL_NT>(v, smem, tot);
            if (tid < 256 && ex < need && need <= ex + v) {
                bcast[0] = tid;
                bcast[1] = need - ex;
            }
            __syncthreads();
            prefix = (prefix << 8) | static_cast<uint32_t>(bcast[0]);
            need = bcast[1];
            __syncthreads();
        }
    }
    // The e selected items are every candidate below tstar plus the first
    // ``need`` equal to it, in position order; one packed scan (below | equal
    // << 16, unsigned: a field's chunk total reaches at most 32768) gives
    // every thread its first list position: (# below before it) + min(# equal
    // before it, need).
    const uint32_t tstar = kmin + prefix;
    int carry_lt = 0, carry_eq = 0;
    for (int c0 = 0; c0 < n_items; c0 += CHUNK) {
        src.load(c0);
        uint32_t ltf = 0, eqf = 0;
#pragma unroll
        for (int k = 0; k < ITEMS; ++k) {
            if ((src.cand >> k) & 1) {
                if (src.key[k] < tstar) ltf |= 1u << k;
                else if (src.key[k] == tstar) eqf |= 1u << k;
            }
        }
        const uint32_t ltc = __popc(ltf), eqc = __popc(eqf);
        uint32_t tot;
        const uint32_t ex = block_exclusive_scan<SEL_NT, uint32_t>(
            ltc | (eqc << 16), reinterpret_cast<uint32_t*>(smem), tot);
        int er = carry_eq + static_cast<int>(ex >> 16);
        int pos = carry_lt + static_cast<int>(ex & 0xFFFFu) + min(er, need);
#pragma unroll
        for (int k = 0; k < ITEMS; ++k) {
            bool sel = (ltf >> k) & 1;
            if ((eqf >> k) & 1) sel = er++ < need;
            if (sel) {
                if (pos < e) out[pos] = src.slot(k);
                ++pos;
            }
        }
        carry_lt += static_cast<int>(tot & 0xFFFFu);
        carry_eq += static_cast<int>(tot >> 16);
    }
}

// The min(n, N) slots of smallest (ts, slot) of each head, ascending, then -1
// up to N.  A commit of N tokens evicts only from these: with r refreshed
// slots and u unmatched tokens (r + u <= N), each of the e <= u evicted slots
// has fewer than e non-refreshed and at most r refreshed slots before it in
// (ts, slot) order.  The list depends on nothing but the timestamps and
// n_valid, so it can be found while the step's attention runs.
__global__ __launch_bounds__(SEL_NT) void tc_order_kernel(const int32_t* __restrict__ ts_all,
                                                          const int32_t* __restrict__ n_valid, int cap,
                                                          int N, int32_t* __restrict__ order) {
    __shared__ int smem[SEL_NT / kWave];
    __shared__ uint32_t red[2 * (SEL_NT / kWave)];
    __shared__ int hist[256];
    __shared__ int bcast[2];
    const int h = blockIdx.x, tid = threadIdx.x;
    const int n = clamp_n(n_valid, h, cap);
    const int m = min(n, N);
    int32_t* out = order + static_cast<size_t>(h) * N;
    if (m < n) {
        SlotRange src(ts_all + static_cast<size_t>(h) * cap, nullptr, n);
        select_smallest(src, n, m, out, smem, red, hist, bcast);
    } else {
        for (int i = tid; i < m; i += SEL_NT) out[i] = i;
    }
    for (int i = m + tid; i < N; i += SEL_NT) out[i] = -1;
}

hipError_t launch_tc_order(const int32_t* ts, const int32_t* n_valid, int H, int cap, int N, int32_t* order,
                           hipStream_t s) {
    if (H == 0 || N == 0) return hipSuccess;
    timer_begin("tempcache_order", s);
    hipLaunchKernelGGL(tc_order_kernel, dim3(H), dim3(SEL_NT), 0, s, ts, n_valid, cap, N, order);
    timer_end(s);
    return hipGetLastError();
}

// LDSC: the claim table (one int per slot) and the refreshed bitmap live in
// LDS (dynamic, cap <= kLdsClaimSlots); otherwise in the workspace.
// LDSG (mean merge): the group sizes, then offsets, of the chunk's tokens
// also live in LDS, after the bitmap; otherwise in the workspace.
template <bool LDSC, bool LDSG>
__global__ __launch_bounds__(SEL_NT) void tc_select_kernel(const TcSelectParams p) {
    extern __shared__ int dyn_lds[];
    __shared__ int smem[SEL_NT / kWave];
    __shared__ uint32_t red[2 * (SEL_NT / kWave)];
    __shared__ int hist[256];
    __shared__ int bcast[2];
    const int h = blockIdx.x, tid = threadIdx.x;
    const int cap = p.cap, N = p.N;
    const int n = clamp_n(p.n_valid, h, cap);
    const int words = (cap + 31) / 32;
    const int32_t* best = p.best + static_cast<size_t>(h) * N;
    const float* cosv = p.cosv + static_cast<size_t>(h) * N;
    int32_t* claim;
    uint32_t* refr;
    if constexpr (LDSC) {
        claim = dyn_lds;
        refr = reinterpret_cast<uint32_t*>(dyn_lds + cap);
    } else {
        claim = p.claim + static_cast<size_t>(h) * cap;
        refr = p.refreshed + static_cast<size_t>(h) * words;
    }
    const int32_t* ts = p.ts + static_cast<size_t>(h) * cap;
    int32_t* upos = p.upos + static_cast<size_t>(h) * N;
    int32_t* ev = p.ev + static_cast<size_t>(h) * N;
    int32_t* dest = p.dest + static_cast<size_t>(h) * N;

    // Token data are held in registers, TOK_ITEMS consecutive tokens per
    // thread; with N <= TOK_CHUNK (one chunk) every phase reuses one load.
    // Each phase issues all its loads before its first store, so the round
    // trips overlap (the stores could alias the loaded arrays).  Loads take
    // clamped indices and are masked afterwards: a load under a branch gets
    // its own wait, and the round trips would run one after another.
    int bi[TOK_ITEMS], up[TOK_ITEMS];
    float ci[TOK_ITEMS];
    int tok_c0 = -1;
    auto load_tok = [&](int c0) __attribute__((always_inline)) {
        if (tok_c0 == c0) return;
        tok_c0 = c0;
        const int base = c0 + tid * TOK_ITEMS;
#pragma unroll
        for (int k = 0; k < TOK_ITEMS; ++k) bi[k] = best[min(base + k, N - 1)];
#pragma unroll
        for (int k = 0; k < TOK_ITEMS; ++k) ci[k] = cosv[min(base + k, N - 1)];
#pragma unroll
        for (int k = 0; k < TOK_ITEMS; ++k)
            if (base + k >= N) {
                bi[k] = -1;
                ci[k] = 0.f;
            }
    };

    const bool merge = p.grp_cnt != nullptr;                  // uniform
    int32_t* gcnt_out = merge ? p.grp_cnt + static_cast<size_t>(h) * N : nullptr;
    int32_t* gpos = merge ? p.grp_pos + static_cast<size_t>(h) * N : nullptr;
    int32_t* gcnt;                       // group sizes (in LDS: offsets after the scan)
    if constexpr (LDSG) gcnt = dyn_lds + (LDSC ? cap + words : 0);
    else gcnt = gcnt_out;
    // a matched token's position in its group: in registers when the tokens
    // fit one chunk, else in the workspace
    int gp[TOK_ITEMS];

    // 1. claims.  Only the entries of matched slots are reset, so the claim
    //    array never needs a full clear.
    for (int w = tid; w < (n + 31) / 32; w += SEL_NT) refr[w] = 0u;
    if (merge)
        for (int i = tid; i < N; i += SEL_NT) gcnt[i] = 0;
    for (int c0 = 0; c0 < N; c0 += TOK_CHUNK) {
        load_tok(c0);
#pragma unroll
        for (int k = 0; k < TOK_ITEMS; ++k)
            if (is_matched(bi[k], ci[k], n, p.tau)) claim[bi[k]] = -1;
    }
    __syncthreads();
    for (int c0 = 0; c0 < N; c0 += TOK_CHUNK) {
        load_tok(c0);
        const int base = c0 + tid * TOK_ITEMS;
#pragma unroll
        for (int k = 0; k < TOK_ITEMS; ++k)
            if (is_matched(bi[k], ci[k], n, p.tau)) atomicMax(&claim[bi[k]], base + k);
    }
    __syncthreads();

    // 2. tokens: matched ones get their slot (winner) or -1 (dropped); the
    //    unmatched are ranked in token order.  One scan carries both counts:
    //    unmatched in the low 16 bits, winners (= refreshed slots) above.
    int u = 0, refreshed = 0;
    for (int c0 = 0; c0 < N; c0 += TOK_CHUNK) {
        load_tok(c0);
        const int base = c0 + tid * TOK_ITEMS;
        int cl[TOK_ITEMS];
#pragma unroll
        for (int k = 0; k < TOK_ITEMS; ++k) cl[k] = claim[min(max(bi[k], 0), cap - 1)];   // no branch
#pragma unroll
        for (int k = 0; k < TOK_ITEMS; ++k)
            if (!(base + k < N && is_matched(bi[k], ci[k], n, p.tau))) cl[k] = -2;
        int local = 0, wins = 0;
#pragma unroll
        for (int k = 0; k < TOK_ITEMS; ++k) {
            const int i = base + k;
            if (i >= N) continue;
            if (cl[k] == -2) {
                ++local;
            } else {
                const bool win = cl[k] == i;
                if (win) atomicOr(&refr[bi[k] >> 5], 1u << (bi[k] & 31));
                wins += win;
                dest[i] = win ? bi[k] : -1;
                // mean merge: the token joins the group of its slot's winner
                if (merge) {
                    gp[k] = atomicAdd(&gcnt[cl[k]], 1);
                    if (N > TOK_CHUNK) gpos[i] = gp[k];
                }
            }
        }
        int total;
        const int excl = block_exclusive_scan<SEL_NT>(local | (wins << 16), smem, total);
        int pos = u + (excl & 0xFFFF);
#pragma unroll
        for (int k = 0; k < TOK_ITEMS; ++k) {
            const int i = base + k;
            up[k] = (i < N && cl[k] == -2) ? pos++ : -1;
            if (i < N && N > TOK_CHUNK) upos[i] = up[k];
        }
        u += total & 0xFFFF;
        refreshed += total >> 16;
    }
    __syncthreads();                    // the refreshed bitmap is complete

    // 2b. mean merge: group offsets (a scan of the group sizes in token
    //     order), then every matched token is placed in its group
    if (merge) {
        int32_t* goff_out = p.grp_off + static_cast<size_t>(h) * N;
        int32_t* gmem = p.grp_mem + static_cast<size_t>(h) * N;
        int carry = 0;
        for (int c0 = 0; c0 < N; c0 += TOK_CHUNK) {
            const int base = c0 + tid * TOK_ITEMS;
            int cn[TOK_ITEMS], local = 0;
#pragma unroll
            for (int k = 0; k < TOK_ITEMS; ++k) {
                cn[k] = (base + k < N) ? gcnt[base + k] : 0;
                local += cn[k];
            }
            int total;
            int pos = carry + block_exclusive_scan<SEL_NT>(local, smem, total);
            // each thread rewrites only its own tokens' entries: in LDS the
            // sizes become offsets (both go to the workspace for the scatter)
#pragma unroll
            for (int k = 0; k < TOK_ITEMS; ++k) {
                if (base + k < N) {
                    if constexpr (LDSG) {
                        gcnt_out[base + k] = cn[k];
                        gcnt[base + k] = pos;
                    }
                    goff_out[base + k] = pos;
                }
                pos += cn[k];
            }
            carry += total;
        }
        __syncthreads();
        for (int c0 = 0; c0 < N; c0 += TOK_CHUNK) {
            load_tok(c0);
            const int base = c0 + tid * TOK_ITEMS;
            // the claim and offset reads take clamped indices (no branch), so
            // each kind's reads are all in flight together
            int wk[TOK_ITEMS], ok[TOK_ITEMS];
#pragma unroll
            for (int k = 0; k < TOK_ITEMS; ++k) wk[k] = claim[min(max(bi[k], 0), cap - 1)];
#pragma unroll
            for (int k = 0; k < TOK_ITEMS; ++k) {
                const int w = min(max(wk[k], 0), N - 1);
                ok[k] = LDSG ? gcnt[w] : goff_out[w];
            }
            if (N > TOK_CHUNK) {                        // uniform: positions from the workspace
#pragma unroll
                for (int k = 0; k < TOK_ITEMS; ++k) gp[k] = gpos[min(base + k, N - 1)];
            }
#pragma unroll
            for (int k = 0; k < TOK_ITEMS; ++k) {
                const int i = base + k;
                if (i < N && is_matched(bi[k], ci[k], n, p.tau)) gmem[ok[k] + gp[k]] = i;
            }
        }
    }

    const int e = max(0, n + u - cap);
    const int appended = u - e;

    // 3. the e oldest non-refreshed slots (ties: lower slot), ascending:
    //    among the precomputed candidates when given, else among all slots
    if (e > 0) {
        if (p.order) {
            SlotList src(p.order + static_cast<size_t>(h) * N, ts, refr, min(n, N), n);
            select_smallest(src, min(n, N), e, ev, smem, red, hist, bcast);
        } else {
            SlotRange src(ts, refr, n);
            select_smallest(src, n, e, ev, smem, red, hist, bcast);
        }
    }
    __syncthreads();

    // 4. unmatched tokens: appended slots first, then the evicted ones
    for (int c0 = 0; c0 < N; c0 += TOK_CHUNK) {
        const int base = c0 + tid * TOK_ITEMS;
        if (N > TOK_CHUNK) {
#pragma unroll
            for (int k = 0; k < TOK_ITEMS; ++k) up[k] = (base + k < N) ? upos[base + k] : -1;
        }
        int dst[TOK_ITEMS], evk[TOK_ITEMS];
#pragma unroll
        for (int k = 0; k < TOK_ITEMS; ++k)         // clamped: every load in flight at once
            evk[k] = ev[min(max(up[k] - appended, 0), N - 1)];
#pragma unroll
        for (int k = 0; k < TOK_ITEMS; ++k)
            dst[k] = up[k] < 0 ? -2 : (up[k] < appended ? n + up[k] : evk[k]);
#pragma unroll
        for (int k = 0; k < TOK_ITEMS; ++k)
            if (dst[k] != -2) dest[base + k] = (dst[k] >= 0 && dst[k] < cap) ? dst[k] : -1;
    }
    if (p.evicted)
        for (int k = tid; k < N; k += SEL_NT)
            p.evicted[static_cast<size_t>(h) * N + k] = (k < e) ? ev[k] : -1;
    if (tid == 0) {
        if (p.counts) {
            int32_t* c = p.counts + static_cast<size_t>(h) * 5;
            c[0] = N - u;
            c[1] = refreshed;
            c[2] = (N - u) - refreshed;
            c[3] = appended;
            c[4] = e;
        }
        p.n_valid[h] = n + appended;
    }
}

hipError_t launch_tc_select(const TcSelectParams& p, hipStream_t s) {
    if (p.H == 0) return hipSuccess;
    timer_begin("tempcache_select", s);
    const bool ldsc = p.cap <= kLdsClaimSlots;
    const size_t claim_bytes = ldsc ? (static_cast<size_t>(p.cap) + (p.cap + 31) / 32) * 4 : 0;
    const size_t grp_bytes = static_cast<size_t>(p.N) * 4;
    const bool ldsg = p.grp_cnt != nullptr && claim_bytes + grp_bytes <= kSelectDynLds;
    const size_t bytes = claim_bytes + (ldsg ? grp_bytes : 0);
    if (ldsc && ldsg)
        hipLaunchKernelGGL((tc_select_kernel<true, true>), dim3(p.H), dim3(SEL_NT), bytes, s, p);
    else if (ldsc)
        hipLaunchKernelGGL((tc_select_kernel<true, false>), dim3(p.H), dim3(SEL_NT), bytes, s, p);
    else if (ldsg)
        hipLaunchKernelGGL((tc_select_kernel<false, true>), dim3(p.H), dim3(SEL_NT), bytes, s, p);
    else
        hipLaunchKernelGGL((tc_select_kernel<false, false>), dim3(p.H), dim3(SEL_NT), 0, s, p);
    timer_end(s);
    return hipGetLastError();
}

// ------------------------------------------------------------------ row scatter
namespace {
constexpr int kGroupLanes = 16;                       // lanes per written token
constexpr int kScatterTokensPerBlock = 256 / kGroupLanes;   // tokens per scatter block

// One lane's share of a d-wide row: D/16 consecutive elements, moved as
// 8, 16 or 32 bytes (the rows are 16-byte aligned).
template <typename T, int D>
struct LaneRow {
    static constexpr int EPL = D / kGroupLanes;
    static constexpr int W = EPL * static_cast<int>(sizeof(T)) / 4;     // 32-bit words
    static_assert(W == 2 || W == 4 || W == 8, "lane share");
    uint32_t w[W];
    __device__ __forceinline__ void load(const T* row, int gl) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(row) + gl * W;
        if constexpr (W == 2) {
            const uint2 a = *reinterpret_cast<const uint2*>(p);
            w[0] = a.x; w[1] = a.y;
        } else {
#pragma unroll
            for (int q = 0; q < W / 4; ++q) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(p + 4 * q);
                w[4 * q] = a[0]; w[4 * q + 1] = a[1]; w[4 * q + 2] = a[2]; w[4 * q + 3] = a[3];
            }
        }
    }
    __device__ __forceinline__ void store(T* row, int gl) const {
        uint32_t* p = reinterpret_cast<uint32_t*>(row) + gl * W;
        if constexpr (W == 2) {
            *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
        } else {
#pragma unroll
            for (int q = 0; q < W / 4; ++q)
                *reinterpret_cast<u32x4*>(p + 4 * q) = u32x4{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]};
        }
    }
    __device__ __forceinline__ float get(int e) const {
        if constexpr (sizeof(T) == 2) return __uint_as_float((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
        else return __uint_as_float(w[e]);
    }
    __device__ __forceinline__ void set(int e, float x) {
        if constexpr (sizeof(T) == 2) {
            const uint32_t b = f32_to_bf16(x);
            w[e >> 1] = (e & 1) ? ((w[e >> 1] & 0xFFFFu) | (b << 16)) : ((w[e >> 1] & 0xFFFF0000u) | b);
        } else {
            w[e] = __float_as_uint(x);
        }
    }
};
}  // namespace

// Sixteen lanes per current token (four tokens per wave): a written token's
// key and value rows move to its slot, with its id, the step as timestamp and
// the key's norm.
template <typename T, int D>
__global__ __launch_bounds__(256) void tc_scatter_kernel(
    const int32_t* __restrict__ dest, const T* __restrict__ kc, const T* __restrict__ vc,
    const uint16_t* __restrict__ kids, int32_t step, T* __restrict__ ck, T* __restrict__ cv,
    uint16_t* __restrict__ cids, int32_t* __restrict__ cts, float* __restrict__ cnorm, int N,
    int cap) {
    using R = LaneRow<T, D>;
    const int h = blockIdx.y;
    const int gl = threadIdx.x % kGroupLanes;
    const int i = blockIdx.x * kScatterTokensPerBlock + threadIdx.x / kGroupLanes;
    if (i >= N) return;                                  // group uniform
    const size_t ti = static_cast<size_t>(h) * N + i;
    const int d = dest[ti];
    if (d < 0 || d >= cap) return;                       // group uniform
    const size_t si = static_cast<size_t>(h) * cap + d;
    R kr, vr;
    kr.load(kc + ti * D, gl);
    vr.load(vc + ti * D, gl);
    kr.store(ck + si * D, gl);
    vr.store(cv + si * D, gl);
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < R::EPL; ++e) sq = __builtin_fmaf(kr.get(e), kr.get(e), sq);
#pragma unroll
    for (int off = kGroupLanes / 2; off >= 1; off >>= 1) sq += __shfl_xor(sq, off);
    if (gl == 0) {
        cids[si] = kids[ti];
        cts[si] = step;
        cnorm[si] = __builtin_sqrtf(sq);
    }
}

hipError_t launch_tc_scatter(bool bf16, int d, int H, int N, int cap, const int32_t* dest,
                             const void* k_cur, const void* v_cur, const uint16_t* kcur_ids,
                             int32_t step, void* ck, void* cv, uint16_t* cids, int32_t* cts,
                             float* cnorm, hipStream_t s) {
    if (H == 0 || N == 0) return hipSuccess;
    dim3 grid((N + kScatterTokensPerBlock - 1) / kScatterTokensPerBlock, H);
    timer_begin("tempcache_scatter", s);
#define FASTAR_SCATTER(T, DD)                                                                     \
    hipLaunchKernelGGL((tc_scatter_kernel<T, DD>), grid, dim3(256), 0, s, dest,                  \
                       static_cast<const T*>(k_cur), static_cast<const T*>(v_cur), kcur_ids, step, \
                       static_cast<T*>(ck), static_cast<T*>(cv), cids, cts, cnorm, N, cap)
    if (bf16) {
        if (d == 64) FASTAR_SCATTER(uint16_t, 64); else FASTAR_SCATTER(uint16_t, 128);
    } else {
        if (d == 64) FASTAR_SCATTER(float, 64); else FASTAR_SCATTER(float, 128);
    }
#undef FASTAR_SCATTER
    timer_end(s);
    return hipGetLastError();
}


// Sixteen lanes per current token with a destination slot (four tokens per
// wave; every cross-lane step stays inside a token's 16 lanes, whose lanes
// are active together).  Lane l of a group owns elements l*D/16 .. of each
// row.  The key row, id, timestamp and norm are written as in the
// replacement scatter.  A token that represents a group of c matched tokens
// sets the slot's value to (m v + sum of the members' values) / (m + c) in
// fp32, members taken in ascending token order, and its group size to m + c;
// any other written token starts a group of one.
template <typename T, int D>
__global__ __launch_bounds__(256) void tc_merge_scatter_kernel(
    const int32_t* __restrict__ dest, const int32_t* __restrict__ gcnt, const int32_t* __restrict__ goff,
    const int32_t* __restrict__ gmem, const T* __restrict__ kc, const T* __restrict__ vc,
    const uint16_t* __restrict__ kids, int32_t step, T* __restrict__ ck, T* __restrict__ cv,
    uint16_t* __restrict__ cids, int32_t* __restrict__ cts, float* __restrict__ cnorm,
    int32_t* __restrict__ ccount, int N, int cap) {
    using R = LaneRow<T, D>;
    constexpr int EPL = R::EPL;
    const int h = blockIdx.y;
    const int gl = threadIdx.x % kGroupLanes;
    const int gb = (threadIdx.x % kWave) - gl;         // the group's first lane in the wave
    const int i = blockIdx.x * kScatterTokensPerBlock + threadIdx.x / kGroupLanes;
    if (i >= N) return;                                  // group uniform
    const size_t ti = static_cast<size_t>(h) * N + i;
    // the group entries are loaded with dest (not after it): one round trip
    const int d = dest[ti];
    const int c = gcnt[ti];
    const int g0 = goff[ti];
    if (d < 0 || d >= cap) return;                       // group uniform
    const size_t si = static_cast<size_t>(h) * cap + d;
    const T* vcur_h = vc + static_cast<size_t>(h) * N * D;

    R kr;
    kr.load(kc + ti * D, gl);
    kr.store(ck + si * D, gl);
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) sq = __builtin_fmaf(kr.get(e), kr.get(e), sq);

    if (c == 0) {                                        // a group of one
        R vr;
        vr.load(vc + ti * D, gl);
        vr.store(cv + si * D, gl);
        if (gl == 0) ccount[si] = 1;
    } else {
        const int m0 = ccount[si];
        const int m = m0 < 1 ? 1 : m0;
        R old;
        old.load(cv + si * D, gl);
        const int32_t* mem = gmem + static_cast<size_t>(h) * N + g0;
        float acc[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = static_cast<float>(m) * old.get(e);
        if (c <= kGroupLanes) {
            // rank each member within the group, then route member r to lane r
            const int mine = gl < c ? mem[gl] : 0x7FFFFFFF;
            int rank = 0;
            for (int t = 0; t < c; ++t) rank += __shfl(mine, gb + t) < mine ? 1 : 0;
            const int slot_lane = gb + (rank < kGroupLanes ? rank : kGroupLanes - 1);
            const int sorted = __builtin_amdgcn_ds_permute(slot_lane * 4, mine);
            constexpr int BT = 4;                        // member rows in flight
            for (int t0 = 0; t0 < c; t0 += BT) {
                R x[BT];
#pragma unroll
                for (int b = 0; b < BT; ++b) {
                    const int t = t0 + b < c ? t0 + b : c - 1;
                    x[b].load(vcur_h + static_cast<size_t>(__shfl(sorted, gb + t)) * D, gl);
                }
#pragma unroll
                for (int b = 0; b < BT; ++b)
                    if (t0 + b < c)
#pragma unroll
                        for (int e = 0; e < EPL; ++e) acc[e] += x[b].get(e);
            }
        } else {
            // large groups: repeatedly take the smallest member above the last
            int last = -1;
            for (int r = 0; r < c; ++r) {
                int cand = 0x7FFFFFFF;
                for (int t = gl; t < c; t += kGroupLanes) {
                    const int x = mem[t];
                    cand = (x > last && x < cand) ? x : cand;
                }
#pragma unroll
                for (int off = kGroupLanes / 2; off >= 1; off >>= 1) {
                    const int o = __shfl_xor(cand, off);
                    cand = o < cand ? o : cand;
                }
                last = cand;
                R x;
                x.load(vcur_h + static_cast<size_t>(last) * D, gl);
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[e] += x.get(e);
            }
        }
        const float tot = static_cast<float>(m + c);
        R out;
#pragma unroll
        for (int e = 0; e < EPL; ++e) out.set(e, acc[e] / tot);
        out.store(cv + si * D, gl);
        if (gl == 0) ccount[si] = m + c;
    }
#pragma unroll
    for (int off = kGroupLanes / 2; off >= 1; off >>= 1) sq += __shfl_xor(sq, off);
    if (gl == 0) {
        cids[si] = kids[ti];
        cts[si] = step;
        cnorm[si] = __builtin_sqrtf(sq);
    }
}

hipError_t launch_tc_merge_scatter(bool bf16, int d, int H, int N, int cap, const int32_t* dest,
                                   const int32_t* grp_cnt, const int32_t* grp_off,
                                   const int32_t* grp_mem, const void* k_cur, const void* v_cur,
                                   const uint16_t* kcur_ids, int32_t step, void* ck, void* cv,
                                   uint16_t* cids, int32_t* cts, float* cnorm, int32_t* ccount,
                                   hipStream_t s) {
    if (H == 0 || N == 0) return hipSuccess;
    dim3 grid((N + kScatterTokensPerBlock - 1) / kScatterTokensPerBlock, H);
    timer_begin("tempcache_merge_scatter", s);
#define FASTAR_MSCATTER(T, DD)                                                                     \
    hipLaunchKernelGGL((tc_merge_scatter_kernel<T, DD>), grid, dim3(256), 0, s,                   \
                       dest, grp_cnt, grp_off, grp_mem, static_cast<const T*>(k_cur),                 \
                       static_cast<const T*>(v_cur), kcur_ids, step, static_cast<T*>(ck),             \
                       static_cast<T*>(cv), cids, cts, cnorm, ccount, N, cap)
    if (bf16) {
        if (d == 64) FASTAR_MSCATTER(uint16_t, 64); else FASTAR_MSCATTER(uint16_t, 128);
    } else {
        if (d == 64) FASTAR_MSCATTER(float, 64); else FASTAR_MSCATTER(float, 128);
    }
#undef FASTAR_MSCATTER
    timer_end(s);
    return hipGetLastError();
}

}  // namespace fastar
