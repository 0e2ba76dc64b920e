// Gathered block attention on the matrix cores, three uses:
//
//  MODE_SA   AnnSA: one block per (head, bucket, 64-query slice).  Queries are
//            the bucket's current-chunk queries, keys the bucket's members of
//            [cache slots ; current chunk] (FAST-AR blog, "3. AnnSA"; summary,
//            "2. Core Components" C).  Softmax attention + log-sum-exp.
//  MODE_CA   AnnCA: one block per (head, frame, 64 consecutive queries); keys
//            are the frame's kept prompt tokens (blog, "2. AnnCA"; summary B).
//  MODE_TOP1 TempCache search: same blocks as SA over old-cache keys only;
//            instead of a softmax each query keeps its best cosine and slot
//            (blog, "1. TempCache"; summary A), then claims the slot.
//
// Layout of the work inside a block (256 threads = 4 waves, wave w owns the
// block's queries 16w..16w+15; lane l serves query l%16 and "lane group"
// g = l/16):
//  * scores are computed transposed, S^T = K Q^T, so that MFMA's output layout
//    (lane holds rows 4g..4g+3 of column l%16) gives every lane a single query
//    and four keys per 16-key block: the row max / sum of the online softmax
//    then need only two cross-lane steps (lanes l, l^16, l^32, l^48), and the
//    probabilities are already laid out as the B operand of O^T = V^T P^T.
//  * K tiles of 64 rows sit row-major in LDS (A operand of S^T, 16 contiguous
//    bytes per lane).  For bf16, V tiles are stored transposed in LDS with the
//    keys of each 32-key group permuted so that lane group g reads its eight
//    keys {4g..4g+3, 16+4g..16+4g+3} as 16 contiguous bytes -- the same keys
//    its probabilities cover.  For fp32 (16x16x4 MFMA) V stays row-major.
//  * Global K/V rows are gathered through the index list with 16-byte loads
//    (16 lanes cover one 256-byte bf16 row), one tile ahead of the compute,
//    and the index list itself two tiles ahead.
#include "common.hpp"
#include "launch.hpp"

namespace fastar {

namespace {

constexpr int KT = 64;            // keys per LDS tile
constexpr float kNegInf = -__builtin_huge_valf();

// Position of key kk (0..63) in a transposed-V row: within each 32-key group,
// keys 4g..4g+3 go to 8g..8g+3 and keys 16+4g..16+4g+3 to 8g+4..8g+7.
__device__ __forceinline__ int vt_pos(int kk) {
    const int grp = kk >> 5, r = kk & 31, quad = r >> 2;
    const int base = quad < 4 ? 8 * quad : 8 * (quad - 4) + 4;
    return grp * 32 + base + (r & 3);
}

template <typename T, int D, int MODE>
struct Tile {
    static constexpr bool BF = sizeof(T) == 2;
    static constexpr bool HAS_V = MODE != MODE_TOP1;
    static constexpr int EPC = 16 / sizeof(T);          // elements per 16-byte chunk
    static constexpr int CPR = D / EPC;                 // chunks per row
    static constexpr int UNITS = (KT / 4) * CPR;        // (4-row quad, chunk) units
    static constexpr int UPT = (UNITS + 255) / 256;     // units per thread
    static constexpr int KSTR = D + (BF ? 8 : 4);            // padded K row (elements)
    static constexpr int VTSTR = KT + 8;                // bf16 transposed V row
    static constexpr int VRSTR = D + 4;                 // fp32 row-major V row
    static constexpr int VSIZE = HAS_V ? (BF ? D * VTSTR : KT * VRSTR) : 1;
};

}  // namespace

template <typename T, int D, int MODE, typename OT>
__global__ __launch_bounds__(256) void attn_kernel(const AttnParams p) {
    using TL = Tile<T, D, MODE>;
    constexpr bool BF = TL::BF;
    constexpr bool HAS_V = TL::HAS_V;
    constexpr int UPT = TL::UPT, CPR = TL::CPR, EPC = TL::EPC;
    constexpr int KSTR = TL::KSTR, VTSTR = TL::VTSTR, VRSTR = TL::VRSTR;
    constexpr int NDB = D / 16;                          // 16-wide output blocks
    constexpr int NKS = BF ? D / 32 : D / 4;             // k-steps of S^T

    __shared__ __align__(16) T Ks[KT * KSTR];
    __shared__ __align__(16) T Vs[TL::VSIZE];
    __shared__ float knorm[MODE == MODE_TOP1 ? KT : 1];
    __shared__ int kslot[MODE == MODE_TOP1 ? KT : 1];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;

    // ---------------------------------------------------------------- work
    int h, q_count, nk, na = 0, qbase = 0;
    const int32_t* qlist = nullptr;
    const int32_t* klist;
    if constexpr (MODE == MODE_CA) {
        h = blockIdx.z;
        const int f = blockIdx.y, c = blockIdx.x;
        qbase = f * p.frame_len + c * kQTile;
        q_count = min(kQTile, p.frame_len - c * kQTile);
        nk = p.ca_cnt[h * p.F + f];
        klist = p.ca_idx + (static_cast<size_t>(h) * p.F + f) * p.L;
    } else {
        h = blockIdx.y;
        const int item = blockIdx.x;
        const int B = p.B;
        const int32_t* wt = p.wt + static_cast<size_t>(h) * (B + 1);
        if (item >= wt[B]) return;
        int lo = 0, hi = B - 1;                 // last bucket with wt[b] <= item
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (wt[mid] <= item) lo = mid; else hi = mid - 1;
        }
        const int b = lo;
        const int32_t* qo = p.qoff + static_cast<size_t>(h) * (B + 1);
        const int qs = qo[b] + (item - wt[b]) * kQTile;
        q_count = min(kQTile, qo[b + 1] - qs);
        qlist = p.qperm + static_cast<size_t>(h) * p.qperm_stride + qs;
        const int32_t* ko = p.koff + static_cast<size_t>(h) * (B + 1);
        nk = ko[b + 1] - ko[b];
        klist = p.kperm + static_cast<size_t>(h) * p.kperm_stride + ko[b];
        na = clamp_n(p.n_valid, h, p.cap);
    }

    const int ql = w * 16 + c16;
    const bool qvalid = ql < q_count;
    const bool wave_active = w * 16 < q_count;
    int qrow = 0;
    if (qvalid) qrow = (MODE == MODE_CA) ? qbase + ql : qlist[ql];

    const T* qh = static_cast<const T*>(p.q) + static_cast<size_t>(h) * p.Nq * D;
    const T* ka = static_cast<const T*>(p.ka) + static_cast<size_t>(h) * p.a_rows * D;
    const T* va = HAS_V ? static_cast<const T*>(p.va) + static_cast<size_t>(h) * p.a_rows * D : nullptr;
    const T* kb = p.kb ? static_cast<const T*>(p.kb) + static_cast<size_t>(h) * p.b_rows * D : nullptr;
    const T* vb = (HAS_V && p.vb) ? static_cast<const T*>(p.vb) + static_cast<size_t>(h) * p.b_rows * D : nullptr;

    // ---------------------------------------------------------------- Q fragments
    // B operand of S^T: lane holds Q[query l%16][k-slice of group g].
    bf16x8_t qf_b[BF ? NKS : 1];
    float qf_f[BF ? 1 : NKS];
    float qsq = 0.f;
    if constexpr (BF) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            uint4 r = make_uint4(0, 0, 0, 0);
            if (qvalid) r = *reinterpret_cast<const uint4*>(qh + static_cast<size_t>(qrow) * D + ks * 32 + 8 * g);
            qf_b[ks] = __builtin_bit_cast(bf16x8_t, r);
            if constexpr (MODE == MODE_TOP1) {
                const uint32_t wv[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float lo = __uint_as_float(wv[i] << 16), hi = __uint_as_float(wv[i] & 0xFFFF0000u);
                    qsq = __builtin_fmaf(lo, lo, qsq);
                    qsq = __builtin_fmaf(hi, hi, qsq);
                }
            }
        }
    } else {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            qf_f[ks] = qvalid ? reinterpret_cast<const float*>(qh)[static_cast<size_t>(qrow) * D + ks * 4 + g] : 0.f;
            if constexpr (MODE == MODE_TOP1) qsq = __builtin_fmaf(qf_f[ks], qf_f[ks], qsq);
        }
    }
    float qnorm = 0.f;
    if constexpr (MODE == MODE_TOP1) {
        qsq += __shfl_xor(qsq, 16);
        qsq += __shfl_xor(qsq, 32);
        qnorm = __builtin_sqrtf(qsq);
    }

    // ---------------------------------------------------------------- tile loads
    int ix[UPT][4];
    int ixk[MODE == MODE_TOP1 ? UPT : 1][4];   // indices of the tile held in kreg
    uint4 kreg[UPT][4];
    uint4 vreg[HAS_V ? UPT : 1][4];

    auto load_idx = [&](int tile) {
#pragma unroll
        for (int k = 0; k < UPT; ++k) {
            const int u = tid + k * 256;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = tile * KT + 4 * (u / CPR) + e;
                ix[k][e] = (u < TL::UNITS && r < nk) ? klist[r] : -1;
            }
        }
    };
    auto load_kv = [&]() {
#pragma unroll
        for (int k = 0; k < UPT; ++k) {
            const int u = tid + k * 256;
            const int chunk = u % CPR;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = ix[k][e];
                uint4 kr = make_uint4(0, 0, 0, 0), vr = make_uint4(0, 0, 0, 0);
                if (j >= 0) {
                    const bool from_a = (MODE == MODE_CA || MODE == MODE_TOP1) || j < na;
                    const size_t row = from_a ? static_cast<size_t>(j) : static_cast<size_t>(j - na);
                    const T* kr_p = (from_a ? ka : kb) + row * D + chunk * EPC;
                    kr = *reinterpret_cast<const uint4*>(kr_p);
                    if constexpr (HAS_V) {
                        const T* vr_p = (from_a ? va : vb) + row * D + chunk * EPC;
                        vr = *reinterpret_cast<const uint4*>(vr_p);
                    }
                }
                kreg[k][e] = kr;
                if constexpr (HAS_V) vreg[k][e] = vr;
                if constexpr (MODE == MODE_TOP1) ixk[k][e] = j;
            }
        }
    };
    auto store_lds = [&]() {
#pragma unroll
        for (int k = 0; k < UPT; ++k) {
            const int u = tid + k * 256;
            if (u >= TL::UNITS) continue;
            const int quad = u / CPR, chunk = u % CPR;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 4 * quad + e;
                *reinterpret_cast<uint4*>(&Ks[row * KSTR + chunk * EPC]) = kreg[k][e];
                if constexpr (HAS_V && !BF)
                    *reinterpret_cast<uint4*>(&Vs[row * VRSTR + chunk * EPC]) = vreg[k][e];
            }
            if constexpr (HAS_V && BF) {
                // 4 keys x 8 dims -> 8 transposed rows of 4 keys (8 bytes each)
                const int pos = vt_pos(4 * quad);
                const uint32_t a0[4] = {vreg[k][0].x, vreg[k][0].y, vreg[k][0].z, vreg[k][0].w};
                const uint32_t a1[4] = {vreg[k][1].x, vreg[k][1].y, vreg[k][1].z, vreg[k][1].w};
                const uint32_t a2[4] = {vreg[k][2].x, vreg[k][2].y, vreg[k][2].z, vreg[k][2].w};
                const uint32_t a3[4] = {vreg[k][3].x, vreg[k][3].y, vreg[k][3].z, vreg[k][3].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // dims 2i (low halves) and 2i+1 (high halves)
                    const uint32_t lo01 = (a0[i] & 0xFFFFu) | (a1[i] << 16);
                    const uint32_t lo23 = (a2[i] & 0xFFFFu) | (a3[i] << 16);
                    const uint32_t hi01 = (a0[i] >> 16) | (a1[i] & 0xFFFF0000u);
                    const uint32_t hi23 = (a2[i] >> 16) | (a3[i] & 0xFFFF0000u);
                    const int d0 = chunk * 8 + 2 * i;
                    *reinterpret_cast<uint2*>(&Vs[d0 * VTSTR + pos]) = make_uint2(lo01, lo23);
                    *reinterpret_cast<uint2*>(&Vs[(d0 + 1) * VTSTR + pos]) = make_uint2(hi01, hi23);
                }
            }
            if constexpr (MODE == MODE_TOP1) {
                // squared norms of the 4 rows: this lane's chunk, then the lanes
                // of the same quad (CPR consecutive lanes)
                float sq[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint4 r = kreg[k][e];
                    const uint32_t wv[4] = {r.x, r.y, r.z, r.w};
                    float s = 0.f;
                    if constexpr (BF) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float lo = __uint_as_float(wv[i] << 16), hi = __uint_as_float(wv[i] & 0xFFFF0000u);
                            s = __builtin_fmaf(lo, lo, s);
                            s = __builtin_fmaf(hi, hi, s);
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float x = __uint_as_float(wv[i]);
                            s = __builtin_fmaf(x, x, s);
                        }
                    }
                    if constexpr (CPR >= 16) {
                        s = group_sum<16>(s);
                        if constexpr (CPR == 32) s += __shfl_xor(s, 16);
                    } else {
                        s = group_sum<8>(s);
                    }
                    sq[e] = s;
                }
                if (chunk == 0) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        knorm[4 * quad + e] = __builtin_sqrtf(sq[e]);
                        kslot[4 * quad + e] = ixk[k][e];
                    }
                }
            }
        }
    };

    // ---------------------------------------------------------------- state
    f32x4 o[HAS_V ? NDB : 1];
#pragma unroll
    for (int i = 0; i < (HAS_V ? NDB : 1); ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kNegInf, l_run = 0.f;             // softmax state (log2 domain)
    float best_c = kNegInf;
    int best_s = 0x7FFFFFFF;                        // TOP1 state

    const int nt = (nk + KT - 1) / KT;
    if (nt > 0) {
        load_idx(0);
        load_kv();
        if (nt > 1) load_idx(1);
    }
#pragma unroll 1
    for (int t = 0; t < nt; ++t) {
        __syncthreads();
        store_lds();
        __syncthreads();
        if (t + 1 < nt) {
            load_kv();
            if (t + 2 < nt) load_idx(t + 2);
        }
        if (!wave_active) continue;

        // ---- S^T = K Q^T for the 4 key blocks of the tile
        f32x4 s[4];
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4) {
            s[kb4] = f32x4{0.f, 0.f, 0.f, 0.f};
            const T* krow = &Ks[(kb4 * 16 + c16) * KSTR];
            if constexpr (BF) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(krow + ks * 32 + 8 * g);
                    s[kb4] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf_b[ks], s[kb4], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const float a = reinterpret_cast<const float*>(krow)[ks * 4 + g];
                    s[kb4] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, qf_f[ks], s[kb4], 0, 0, 0);
                }
            }
        }
        const int kbase = t * KT;

        if constexpr (MODE == MODE_TOP1) {
#pragma unroll
            for (int kb4 = 0; kb4 < 4; ++kb4) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int kk = kb4 * 16 + 4 * g + r;
                    if (kbase + kk < nk) {
                        const float den = qnorm * knorm[kk];
                        const float c = den > 0.f ? s[kb4][r] / den : 0.f;
                        if (c > best_c) { best_c = c; best_s = kslot[kk]; }
                    }
                }
            }
        } else {
            // ---- online softmax (log2 domain), one query per lane
            float tmax = kNegInf;
#pragma unroll
            for (int kb4 = 0; kb4 < 4; ++kb4) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int kk = kb4 * 16 + 4 * g + r;
                    const float v = (kbase + kk < nk) ? s[kb4][r] * p.scale_log2 : kNegInf;
                    s[kb4][r] = v;
                    tmax = fmaxf(tmax, v);
                }
            }
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float m_new = fmaxf(m_run, tmax);
            const float m_use = (m_new == kNegInf) ? 0.f : m_new;
            const float alpha = (m_run == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_use);
            float psum = 0.f;
#pragma unroll
            for (int kb4 = 0; kb4 < 4; ++kb4) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float e = __builtin_amdgcn_exp2f(s[kb4][r] - m_use);
                    s[kb4][r] = e;
                    psum += e;
                }
            }
            l_run = l_run * alpha + psum;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] *= alpha;

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
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
                            &Vs[(db * 16 + c16) * VTSTR + kg * 32 + 8 * g]);
                        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o[db], 0, 0, 0);
                    }
                }
            } else {
#pragma unroll
                for (int kb4 = 0; kb4 < 4; ++kb4) {
#pragma unroll
                    for (int st = 0; st < 4; ++st) {
                        const float* vrow = reinterpret_cast<const float*>(&Vs[(kb4 * 16 + 4 * g + st) * VRSTR]);
#pragma unroll
                        for (int db = 0; db < NDB; ++db)
                            o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vrow[db * 16 + c16], s[kb4][st], o[db], 0, 0, 0);
                    }
                }
            }
        }
    }

    // ---------------------------------------------------------------- epilogue
    if constexpr (MODE == MODE_TOP1) {
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
            const float oc = __shfl_xor(best_c, off);
            const int os = __shfl_xor(best_s, off);
            if (oc > best_c || (oc == best_c && os < best_s)) { best_c = oc; best_s = os; }
        }
        if (qvalid && g == 0) {
            const bool found = best_s != 0x7FFFFFFF;
            const size_t qi = static_cast<size_t>(h) * p.Nq + qrow;
            p.best[qi] = found ? best_s : -1;
            p.bcos[qi] = found ? best_c : kNegInf;
            if (found && best_c >= p.tau)
                atomicMax(&p.claim[static_cast<size_t>(h) * p.cap + best_s], qrow);
        }
    } else {
        float l_tot = l_run + __shfl_xor(l_run, 16);
        l_tot += __shfl_xor(l_tot, 32);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        if (qvalid) {
            OT* orow = static_cast<OT*>(p.out) + (static_cast<size_t>(h) * p.Nq + qrow) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const f32x4 v = o[db] * inv;
                if constexpr (sizeof(OT) == 4) {
                    *reinterpret_cast<float4*>(orow + db * 16 + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
                } else {
                    const uint32_t lo = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
                    const uint32_t hi = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
                    *reinterpret_cast<uint2*>(orow + db * 16 + 4 * g) = make_uint2(lo, hi);
                }
            }
            if (MODE == MODE_SA && p.lse && g == 0)
                p.lse[static_cast<size_t>(h) * p.Nq + qrow] =
                    l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * 0.69314718055994531f : kNegInf;
        }
    }
}

template <typename T, int D, int MODE, typename OT>
static void attn_go(int H, const AttnParams& p, hipStream_t s) {
    dim3 grid;
    if constexpr (MODE == MODE_CA)
        grid = dim3((p.frame_len + kQTile - 1) / kQTile, p.F, H);
    else
        grid = dim3(p.max_items, H);
    if (grid.x == 0 || grid.y == 0 || grid.z == 0) return;
    hipLaunchKernelGGL((attn_kernel<T, D, MODE, OT>), grid, dim3(256), 0, s, p);
}

template <int MODE>
static void attn_dispatch(bool bf16, int d, bool out_bf16, int H, const AttnParams& p, hipStream_t s) {
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

hipError_t launch_attn(int mode, bool bf16, int d, bool out_bf16, int H, const AttnParams& p,
                       hipStream_t s) {
    if (H == 0) return hipSuccess;
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
