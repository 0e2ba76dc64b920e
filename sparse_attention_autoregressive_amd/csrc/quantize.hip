// Quantization bucket ids: each vector goes to its nearest codeword of its
// head's codebook (FAST-AR summary, "2. Core Components", parts A and B name
// quantization as the alternative to LSH for the shared bucket space).
//
//   id(x) = argmin_c |x - c|^2 = argmax_c <x, c> - |c|^2 / 2   (lowest c on ties)
//
// The inner products X C^T are a dense contraction, so they run on the matrix
// cores: for fp32 vectors fp32 v_mfma_f32_16x16x4f32 (below); for bf16
// vectors bf16 MFMA on an exact three-way split of the codebook
// (quantize_bf16_kernel).  Scores are formed transposed, S^T = C X^T,
// so that each lane holds one vector (column) and four codewords (rows) of
// every 16 x 16 block and keeps a running best over its codewords; the four
// lane groups of a vector merge at the end.  The contraction index is
// permuted consistently on both operands -- lane group g sums dimensions
// g*D/4 .. (g+1)*D/4-1 -- so every lane reads contiguous runs of both.
//
// fp32 vectors: a block of 4 waves takes 64 vectors (16 per wave, held in
// registers) and streams the codebook through LDS 64 codewords at a time, with each
// codeword's |c|^2 / 2 (padding codewords past B get +inf).  LDS rows are
// padded by 4 floats so the 16 rows one quarter-wave reads fall on distinct
// banks.  The same pass can write |x|.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace fastar {

// Up to kHashBatch token sets quantized with the same codebook in one launch
// (grid z = set), like the hash's batched form.
struct QzSets {
    const void* x[kHashBatch];
    int N[kHashBatch];
    uint16_t* ids[kHashBatch];
    float* norms[kHashBatch];
};

namespace {
constexpr int QZ_CW = 64;        // codewords per LDS chunk
constexpr int QZ_TOK = 64;       // vectors per block
constexpr int QZ_NB = 4;         // 16-codeword blocks whose MFMA chains interleave
}  // namespace

template <typename T, int D>
__global__ __launch_bounds__(256) void quantize_kernel(const QzSets sets, const float* __restrict__ cb, int B) {
    constexpr int DG = D / 4;                  // dimensions per lane group
    constexpr int STR = D + 4;                 // LDS row stride (floats)
    __shared__ __align__(16) float cs[QZ_CW * STR];
    __shared__ float hn[QZ_CW];
    const T* __restrict__ x = static_cast<const T*>(sets.x[blockIdx.z]);
    const int N = sets.N[blockIdx.z];
    uint16_t* __restrict__ ids = sets.ids[blockIdx.z];
    float* __restrict__ norms = sets.norms[blockIdx.z];
    if (blockIdx.x * QZ_TOK >= N) return;      // block uniform
    const int h = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int tok = blockIdx.x * QZ_TOK + w * 16 + c16;
    const bool valid = tok < N;

    // this lane's slice of its vector: dimensions g*DG .. g*DG + DG-1
    float xv[DG];
    {
        const T* row = x + (static_cast<size_t>(h) * N + (valid ? tok : 0)) * D + g * DG;
#pragma unroll
        for (int e = 0; e < DG; e += 8) {
            float v[8];
            load8_f32(row + e, v);
#pragma unroll
            for (int k = 0; k < 8; ++k) xv[e + k] = valid ? v[k] : 0.f;
        }
    }

    const float* cbh = cb + static_cast<size_t>(h) * B * D;
    float best = -__builtin_huge_valf();
    int bidx = 0x7FFFFFFF;
    for (int c0 = 0; c0 < B; c0 += QZ_CW) {
        __syncthreads();                       // the previous chunk is consumed
        // stage 64 codewords (16-byte pieces; rows past B are zero)
        for (int pidx = tid; pidx < QZ_CW * (D / 4); pidx += 256) {
            const int r = pidx / (D / 4), q = pidx % (D / 4);
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c0 + r < B) v = *reinterpret_cast<const float4*>(cbh + static_cast<size_t>(c0 + r) * D + 4 * q);
            *reinterpret_cast<float4*>(&cs[r * STR + 4 * q]) = v;
        }
        __syncthreads();
        // |c|^2 / 2 of each staged codeword (+inf past B): 4 lanes per row
        for (int r = tid >> 2; r < QZ_CW; r += 64) {
            const int part = tid & 3;
            float sq = 0.f;
#pragma unroll 8
            for (int k = part * DG; k < (part + 1) * DG; ++k) sq = __builtin_fmaf(cs[r * STR + k], cs[r * STR + k], sq);
            sq += __shfl_xor(sq, 1);
            sq += __shfl_xor(sq, 2);
            if (part == 0) hn[r] = c0 + r < B ? 0.5f * sq : __builtin_huge_valf();
        }
        __syncthreads();
        // four 16-codeword blocks at a time: four independent MFMA chains
#pragma unroll 1
        for (int blk0 = 0; blk0 < QZ_CW / 16; blk0 += QZ_NB) {
            f32x4 acc[QZ_NB];
            const float* crow[QZ_NB];
#pragma unroll
            for (int b = 0; b < QZ_NB; ++b) {
                acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
                crow[b] = &cs[((blk0 + b) * 16 + c16) * STR + g * DG];
            }
#pragma unroll
            for (int e = 0; e < DG; e += 4) {
                float4 a[QZ_NB];
#pragma unroll
                for (int b = 0; b < QZ_NB; ++b) a[b] = *reinterpret_cast<const float4*>(crow[b] + e);
#pragma unroll
                for (int b = 0; b < QZ_NB; ++b) acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[b].x, xv[e], acc[b], 0, 0, 0);
#pragma unroll
                for (int b = 0; b < QZ_NB; ++b) acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[b].y, xv[e + 1], acc[b], 0, 0, 0);
#pragma unroll
                for (int b = 0; b < QZ_NB; ++b) acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[b].z, xv[e + 2], acc[b], 0, 0, 0);
#pragma unroll
                for (int b = 0; b < QZ_NB; ++b) acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[b].w, xv[e + 3], acc[b], 0, 0, 0);
            }
            // lane holds codewords (blk0+b)*16 + 4g + r (ascending in b, r) of its vector
#pragma unroll
            for (int b = 0; b < QZ_NB; ++b) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int cl = (blk0 + b) * 16 + 4 * g + r;
                    const float sc = acc[b][r] - hn[cl];
                    if (sc > best) {
                        best = sc;
                        bidx = c0 + cl;
                    }
                }
            }
        }
    }
    // merge the four lane groups (each saw a disjoint quarter of the codewords)
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
        const float ob = __shfl_xor(best, off);
        const int oi = __shfl_xor(bidx, off);
        if (ob > best || (ob == best && oi < bidx)) {
            best = ob;
            bidx = oi;
        }
    }
    float sq = 0.f;
    if (norms) {
#pragma unroll
        for (int e = 0; e < DG; ++e) sq = __builtin_fmaf(xv[e], xv[e], sq);
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
    }
    if (valid && g == 0) {
        ids[static_cast<size_t>(h) * N + tok] = static_cast<uint16_t>(bidx);
        if (norms) norms[static_cast<size_t>(h) * N + tok] = __builtin_sqrtf(sq);
    }
}

// bf16 vectors: the contraction runs on v_mfma_f32_16x16x32_bf16 with each
// fp32 codebook element split exactly into three bf16 terms (hi + mid + lo,
// successive 8-bit slices of the significand by truncation), as the hash does
// with its planes: every product is exact and the three fp32-accumulated
// sums, added smallest first, carry one fp32 dot product's error.  A block of
// 4 waves takes 64 * QZB_GPW vectors (QZB_GPW 16-vector groups per wave, their
// 16-byte loads all in flight); the codebook streams through LDS 64 codewords at a
// time as the three bf16 parts, with |c|^2 / 2 summed in fp32 from the fp32
// values while they are split.  Lane group g supplies dimensions
// 32k + 8g .. 32k + 8g + 7 of k-step k on both operands.
// 16-vector groups per wave of the bf16 kernel (128 vectors per block;
// codebooks above 128 codewords, and any codebook before the resident form
// below): measured 14.2-14.5 us per launch at the Wan-1.3B chunk's 4680 x 12
// vectors and 128 codewords, against 15.6 with four groups and 20.2-20.5 with
// one.
constexpr int QZB_GPW = 2;

template <int D>
__global__ __launch_bounds__(256) void quantize_bf16_kernel(const QzSets sets, const float* __restrict__ cb,
                                                            int B) {
    constexpr int KS = D / 32;
    constexpr int PSTR = D + 8;                // bf16 LDS row stride (elements): 16-byte pad
    constexpr int EPT = D / 4;                 // codebook elements per staging thread
    __shared__ __align__(16) uint16_t cp[3][QZ_CW * PSTR];
    __shared__ __align__(16) float hn[QZ_CW];
    const uint16_t* __restrict__ x = static_cast<const uint16_t*>(sets.x[blockIdx.z]);
    const int N = sets.N[blockIdx.z];
    uint16_t* __restrict__ ids = sets.ids[blockIdx.z];
    float* __restrict__ norms = sets.norms[blockIdx.z];
    if (blockIdx.x * (64 * QZB_GPW) >= N) return;      // block uniform
    const int h = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int i0 = blockIdx.x * (64 * QZB_GPW) + w * 16 * QZB_GPW;

    u32x4 xr[QZB_GPW][KS];
#pragma unroll
    for (int q = 0; q < QZB_GPW; ++q) {
        const int i = i0 + 16 * q + c16;
        const uint16_t* row = x + (static_cast<size_t>(h) * N + (i < N ? i : 0)) * D + g * 8;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            xr[q][k] = u32x4{0u, 0u, 0u, 0u};
            if (i < N) xr[q][k] = *reinterpret_cast<const u32x4*>(row + 32 * k);
        }
    }

    const float* cbh = cb + static_cast<size_t>(h) * B * D;
    float best[QZB_GPW];
    int bidx[QZB_GPW];
#pragma unroll
    for (int q = 0; q < QZB_GPW; ++q) {
        best[q] = -__builtin_huge_valf();
        bidx[q] = 0x7FFFFFFF;
    }
    for (int c0 = 0; c0 < B; c0 += QZ_CW) {
        __syncthreads();                       // the previous chunk is consumed
        // stage 64 codewords as three bf16 parts (rows past B are zero) and
        // their |c|^2 / 2 (+inf past B): thread (r, part) takes D/4 elements
        {
            const int r = tid >> 2, part = tid & 3;
            const bool in = c0 + r < B;
            const float* src = cbh + static_cast<size_t>(c0 + r) * D + part * EPT;
            float sq = 0.f;
#pragma unroll
            for (int e = 0; e < EPT; e += 8) {
                float v[8];
#pragma unroll
                for (int k = 0; k < 8; k += 4) {
                    float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (in) f = *reinterpret_cast<const float4*>(src + e + k);
                    v[k] = f.x; v[k + 1] = f.y; v[k + 2] = f.z; v[k + 3] = f.w;
                }
                uint32_t hw[4], mw[4], lw[4];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    sq = __builtin_fmaf(v[k], v[k], sq);
                    const uint32_t hi = __float_as_uint(v[k]) & 0xFFFF0000u;
                    const float r1 = v[k] - __uint_as_float(hi);
                    const uint32_t mid = __float_as_uint(r1) & 0xFFFF0000u;
                    const uint32_t lo = __float_as_uint(r1 - __uint_as_float(mid)) & 0xFFFF0000u;
                    if ((k & 1) == 0) { hw[k / 2] = hi >> 16; mw[k / 2] = mid >> 16; lw[k / 2] = lo >> 16; }
                    else { hw[k / 2] |= hi; mw[k / 2] |= mid; lw[k / 2] |= lo; }
                }
                const int off = r * PSTR + part * EPT + e;
                *reinterpret_cast<u32x4*>(&cp[0][off]) = u32x4{hw[0], hw[1], hw[2], hw[3]};
                *reinterpret_cast<u32x4*>(&cp[1][off]) = u32x4{mw[0], mw[1], mw[2], mw[3]};
                *reinterpret_cast<u32x4*>(&cp[2][off]) = u32x4{lw[0], lw[1], lw[2], lw[3]};
            }
            sq += __shfl_xor(sq, 1);
            sq += __shfl_xor(sq, 2);
            if (part == 0) hn[r] = in ? 0.5f * sq : __builtin_huge_valf();
        }
        __syncthreads();
#pragma unroll 1
        for (int blk = 0; blk < QZ_CW / 16; ++blk) {
            bf16x8_t a[3][KS];
#pragma unroll
            for (int part = 0; part < 3; ++part)
#pragma unroll
                for (int k = 0; k < KS; ++k)
                    a[part][k] = *reinterpret_cast<const bf16x8_t*>(&cp[part][(blk * 16 + c16) * PSTR + 32 * k + 8 * g]);
            const float4 hb = *reinterpret_cast<const float4*>(&hn[blk * 16 + 4 * g]);
            const float hv[4] = {hb.x, hb.y, hb.z, hb.w};
#pragma unroll
            for (int q = 0; q < QZB_GPW; ++q) {
                f32x4 acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, xr[q][k]);
#pragma unroll
                    for (int part = 0; part < 3; ++part)
                        acc[part] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[part][k], bv, acc[part], 0, 0, 0);
                }
                // lane holds codewords blk*16 + 4g + r (ascending in blk, r) of its vector
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float sc = (acc[0][r] + (acc[1][r] + acc[2][r])) - hv[r];
                    if (sc > best[q]) {
                        best[q] = sc;
                        bidx[q] = c0 + blk * 16 + 4 * g + r;
                    }
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < QZB_GPW; ++q) {
        float bq = best[q];
        int iq = bidx[q];
        // merge the four lane groups (each saw a disjoint quarter of the codewords)
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
            const float ob = __shfl_xor(bq, off);
            const int oi = __shfl_xor(iq, off);
            if (ob > bq || (ob == bq && oi < iq)) {
                bq = ob;
                iq = oi;
            }
        }
        float sq = 0.f;
        if (norms) {
#pragma unroll
            for (int k = 0; k < KS; ++k)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float lo = __uint_as_float(xr[q][k][j] << 16), hi = __uint_as_float(xr[q][k][j] & 0xFFFF0000u);
                    sq = __builtin_fmaf(lo, lo, sq);
                    sq = __builtin_fmaf(hi, hi, sq);
                }
            sq += __shfl_xor(sq, 16);
            sq += __shfl_xor(sq, 32);
        }
        const int i = i0 + 16 * q + c16;
        if (i < N && g == 0) {
            ids[static_cast<size_t>(h) * N + i] = static_cast<uint16_t>(iq);
            if (norms) norms[static_cast<size_t>(h) * N + i] = __builtin_sqrtf(sq);
        }
    }
}

// Codebooks of up to 128 codewords (bf16 vectors): the block stages its
// head's whole codebook, split, once (3 x 128 rows in dynamic LDS) and then
// streams 256-vector tiles of every set of that head through it, blocks of a
// head taking every BPH-th tile.  Each wave holds two 16-vector groups, so
// every codebook fragment read from LDS feeds two MFMAs, and takes the
// codewords two 16-row blocks at a time (rows past B are zero with an
// infinite |c|^2, so an odd block count pads safely): twelve independent
// MFMA chains per step.  A tile's vectors are loaded while the previous
// tile's products run (two register buffers named in alternate steps, so no
// copy waits on a load in flight).
// 8 waves of two groups (two waves per SIMD); measured at the Wan-1.3B
// chunk's two sets: 20.8-21.1 us, against 24.6-25.2 for 4 waves of four
// groups or of two (one wave per SIMD).
#ifndef QZR_WAVES
#define QZR_WAVES 8
#endif
#ifndef QZR_GROUPS
#define QZR_GROUPS 2
#endif
constexpr int QZR_NT = 64 * QZR_WAVES;
constexpr int QZR_GPW = QZR_GROUPS;            // 16-vector groups per wave
constexpr int QZR_TV = QZR_NT / 64 * 16 * QZR_GPW;   // vectors per tile
constexpr int QZR_MAXB = 128;

template <int D>
__global__ __launch_bounds__(QZR_NT)
__attribute__((amdgpu_waves_per_eu(QZR_WAVES >= 8 ? 2 : 1, QZR_WAVES >= 8 ? 2 : 1)))
void quantize_bf16_resident_kernel(const QzSets sets, int nsets,
                                                                        const float* __restrict__ cb, int B,
                                                                        int bph) {
    constexpr int KS = D / 32;
    constexpr int PSTR = D + 8;
    extern __shared__ __align__(16) uint16_t qz_lds[];
    uint16_t* cp0 = qz_lds;
    uint16_t* cp1 = cp0 + QZR_MAXB * PSTR;
    uint16_t* cp2 = cp1 + QZR_MAXB * PSTR;
    float* hn = reinterpret_cast<float*>(cp2 + QZR_MAXB * PSTR);
    const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int nblk2 = ((B + 31) / 32) * 2;              // 16-row blocks, even

    // the head's tiles, set after set
    int tstart[kHashBatch + 1];
    tstart[0] = 0;
#pragma unroll
    for (int s = 0; s < kHashBatch; ++s)
        tstart[s + 1] = tstart[s] + (s < nsets ? (sets.N[s] + QZR_TV - 1) / QZR_TV : 0);
    const int ntiles = tstart[kHashBatch];

    // one tile's vector fragments: this lane's two vectors, 16-byte loads with
    // a clamped row (masked at the write), all in flight together
    struct Tile {
        u32x4 x[QZR_GPW][KS];
        int set, i0;
    };
    auto fetch = [&](Tile& t, int tile) __attribute__((always_inline)) {
        int s = 0;
#pragma unroll
        for (int k = 1; k < kHashBatch; ++k) s += (k < nsets && tile >= tstart[k]) ? 1 : 0;
        t.set = s;
        const int Ns = sets.N[s];
        t.i0 = (tile - tstart[s]) * QZR_TV + w * 16 * QZR_GPW + c16;
        const uint16_t* xs = static_cast<const uint16_t*>(sets.x[s]);
#pragma unroll
        for (int q = 0; q < QZR_GPW; ++q) {
            const uint16_t* row = xs + (static_cast<size_t>(h) * Ns + min(t.i0 + 16 * q, Ns - 1)) * D + g * 8;
#pragma unroll
            for (int k = 0; k < KS; ++k) t.x[q][k] = *reinterpret_cast<const u32x4*>(row + 32 * k);
        }
    };
    auto finish = [&](const Tile& t) __attribute__((always_inline)) {
        const int Ns = sets.N[t.set];
        float best[QZR_GPW];
        int bidx[QZR_GPW];
#pragma unroll
        for (int q = 0; q < QZR_GPW; ++q) {
            best[q] = -__builtin_huge_valf();
            bidx[q] = 0x7FFFFFFF;
        }
#pragma unroll 1
        for (int blk = 0; blk < nblk2; blk += 2) {
            bf16x8_t a[2][3][KS];
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int k = 0; k < KS; ++k) {
                    const int off = ((blk + bb) * 16 + c16) * PSTR + 32 * k + 8 * g;
                    a[bb][0][k] = *reinterpret_cast<const bf16x8_t*>(&cp0[off]);
                    a[bb][1][k] = *reinterpret_cast<const bf16x8_t*>(&cp1[off]);
                    a[bb][2][k] = *reinterpret_cast<const bf16x8_t*>(&cp2[off]);
                }
            f32x4 acc[2][QZR_GPW][3];
#pragma unroll
            for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                for (int q = 0; q < QZR_GPW; ++q)
#pragma unroll
                    for (int part = 0; part < 3; ++part) acc[bb][q][part] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < KS; ++k)
#pragma unroll
                for (int bb = 0; bb < 2; ++bb)
#pragma unroll
                    for (int q = 0; q < QZR_GPW; ++q) {
                        const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, t.x[q][k]);
#pragma unroll
                        for (int part = 0; part < 3; ++part)
                            acc[bb][q][part] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[bb][part][k], bv,
                                                                                      acc[bb][q][part], 0, 0, 0);
                    }
#pragma unroll
            for (int bb = 0; bb < 2; ++bb) {
                const float4 hb = *reinterpret_cast<const float4*>(&hn[(blk + bb) * 16 + 4 * g]);
                const float hv[4] = {hb.x, hb.y, hb.z, hb.w};
#pragma unroll
                for (int q = 0; q < QZR_GPW; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float sc = (acc[bb][q][0][r] + (acc[bb][q][1][r] + acc[bb][q][2][r])) - hv[r];
                        if (sc > best[q]) {
                            best[q] = sc;
                            bidx[q] = (blk + bb) * 16 + 4 * g + r;
                        }
                    }
            }
        }
        float* norms = sets.norms[t.set];
#pragma unroll
        for (int q = 0; q < QZR_GPW; ++q) {
            float bq = best[q];
            int iq = bidx[q];
#pragma unroll
            for (int off = 16; off <= 32; off <<= 1) {
                const float ob = __shfl_xor(bq, off);
                const int oi = __shfl_xor(iq, off);
                if (ob > bq || (ob == bq && oi < iq)) {
                    bq = ob;
                    iq = oi;
                }
            }
            float sq = 0.f;
            if (norms) {
#pragma unroll
                for (int k = 0; k < KS; ++k)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float lo = __uint_as_float(t.x[q][k][j] << 16);
                        const float hi = __uint_as_float(t.x[q][k][j] & 0xFFFF0000u);
                        sq = __builtin_fmaf(lo, lo, sq);
                        sq = __builtin_fmaf(hi, hi, sq);
                    }
                sq += __shfl_xor(sq, 16);
                sq += __shfl_xor(sq, 32);
            }
            const int i = t.i0 + 16 * q;
            if (i < Ns && g == 0) {
                sets.ids[t.set][static_cast<size_t>(h) * Ns + i] = static_cast<uint16_t>(iq);
                if (norms) norms[static_cast<size_t>(h) * Ns + i] = __builtin_sqrtf(sq);
            }
        }
    };

    Tile A, Bt;
    int tile = blockIdx.x;
    if (tile < ntiles) fetch(A, tile);                 // block uniform
    // stage the codebook: thread (row r, quarter part) splits D/4 elements
#pragma unroll
    for (int rp = tid; rp < QZR_MAXB * 4; rp += QZR_NT) {
        const float* cbh = cb + static_cast<size_t>(h) * B * D;
        constexpr int EPT = D / 4;
        const int r = rp >> 2, part = rp & 3;
        const bool in = r < B;
        const float* src = cbh + static_cast<size_t>(min(r, B - 1)) * D + part * EPT;
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < EPT; e += 8) {
            float v[8];
#pragma unroll
            for (int k = 0; k < 8; k += 4) {
                const float4 f = *reinterpret_cast<const float4*>(src + e + k);
                v[k] = in ? f.x : 0.f; v[k + 1] = in ? f.y : 0.f; v[k + 2] = in ? f.z : 0.f; v[k + 3] = in ? f.w : 0.f;
            }
            uint32_t hw[4], mw[4], lw[4];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                sq = __builtin_fmaf(v[k], v[k], sq);
                const uint32_t hi = __float_as_uint(v[k]) & 0xFFFF0000u;
                const float r1 = v[k] - __uint_as_float(hi);
                const uint32_t mid = __float_as_uint(r1) & 0xFFFF0000u;
                const uint32_t lo = __float_as_uint(r1 - __uint_as_float(mid)) & 0xFFFF0000u;
                if ((k & 1) == 0) { hw[k / 2] = hi >> 16; mw[k / 2] = mid >> 16; lw[k / 2] = lo >> 16; }
                else { hw[k / 2] |= hi; mw[k / 2] |= mid; lw[k / 2] |= lo; }
            }
            const int off = r * PSTR + part * EPT + e;
            *reinterpret_cast<u32x4*>(&cp0[off]) = u32x4{hw[0], hw[1], hw[2], hw[3]};
            *reinterpret_cast<u32x4*>(&cp1[off]) = u32x4{mw[0], mw[1], mw[2], mw[3]};
            *reinterpret_cast<u32x4*>(&cp2[off]) = u32x4{lw[0], lw[1], lw[2], lw[3]};
        }
        sq += __shfl_xor(sq, 1);
        sq += __shfl_xor(sq, 2);
        if (part == 0) hn[r] = in ? 0.5f * sq : __builtin_huge_valf();
    }
    __syncthreads();
#pragma unroll 1
    for (; tile < ntiles; tile += 2 * bph) {            // block uniform
        fetch(Bt, min(tile + bph, ntiles - 1));         // past the end: a repeated tile, not written
        finish(A);
        if (tile + bph >= ntiles) break;
        fetch(A, min(tile + 2 * bph, ntiles - 1));
        finish(Bt);
    }
}

hipError_t launch_quantize_batch(int count, const void* const* x, const int* N, uint16_t* const* ids,
                                 float* const* norms, bool bf16, int H, int d, const float* codebook, int B,
                                 hipStream_t s) {
    QzSets sets;
    int used = 0, nmax = 0;
    for (int i = 0; i < count && i < kHashBatch; ++i) {
        if (N[i] == 0) continue;
        sets.x[used] = x[i];
        sets.N[used] = N[i];
        sets.ids[used] = ids[i];
        sets.norms[used] = norms ? norms[i] : nullptr;
        nmax = N[i] > nmax ? N[i] : nmax;
        ++used;
    }
    if (used == 0 || H == 0) return hipSuccess;
    for (int i = used; i < kHashBatch; ++i) {
        sets.x[i] = nullptr;
        sets.N[i] = 0;
        sets.ids[i] = nullptr;
        sets.norms[i] = nullptr;
    }
    timer_begin("ann_quantize", s);
    if (bf16 && B <= QZR_MAXB) {
        int ntiles = 0;
        for (int i = 0; i < used; ++i) ntiles += (sets.N[i] + QZR_TV - 1) / QZR_TV;
        // one block per CU (the staged codebook takes most of its LDS): the
        // head's blocks share its tiles
        const int bph = std::max(1, std::min(ntiles, 256 / std::max(1, H)));
        const int pstr = d + 8;
        const size_t lds = static_cast<size_t>(3 * QZR_MAXB * pstr) * 2 + QZR_MAXB * 4;
        if (d == 64)
            hipLaunchKernelGGL((quantize_bf16_resident_kernel<64>), dim3(bph, H), dim3(QZR_NT), lds, s, sets, used,
                               codebook, B, bph);
        else
            hipLaunchKernelGGL((quantize_bf16_resident_kernel<128>), dim3(bph, H), dim3(QZR_NT), lds, s, sets, used,
                               codebook, B, bph);
    } else if (bf16) {
        const dim3 gb((nmax + 64 * QZB_GPW - 1) / (64 * QZB_GPW), H, used);
        if (d == 64)
            hipLaunchKernelGGL((quantize_bf16_kernel<64>), gb, dim3(256), 0, s, sets, codebook, B);
        else
            hipLaunchKernelGGL((quantize_bf16_kernel<128>), gb, dim3(256), 0, s, sets, codebook, B);
    } else {
        const dim3 grid((nmax + QZ_TOK - 1) / QZ_TOK, H, used);
        if (d == 64)
            hipLaunchKernelGGL((quantize_kernel<float, 64>), grid, dim3(256), 0, s, sets, codebook, B);
        else
            hipLaunchKernelGGL((quantize_kernel<float, 128>), grid, dim3(256), 0, s, sets, codebook, B);
    }
    timer_end(s);
    return hipGetLastError();
}

hipError_t launch_quantize(const void* x, bool bf16, int H, int N, int d, const float* codebook, int B,
                           uint16_t* ids, float* norms, hipStream_t s) {
    return launch_quantize_batch(1, &x, &N, &ids, &norms, bf16, H, d, codebook, B, s);
}

}  // namespace fastar
