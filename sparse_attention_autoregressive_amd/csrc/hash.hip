// Random-hyperplane bucket ids (the LSH that places queries, cache keys,
// current keys and prompt keys in one shared bucket space; FAST-AR summary,
// "2. Core Components", parts A and B):
//
//   id(x) = sum_p [<x, r_p> >= 0] << p
//
// The projections onto the P <= 16 planes are one 16-row matrix-core block per
// 16 vectors (see hash_kernel; bf16 vectors on bf16 MFMA with each plane split
// exactly into three bf16 terms).  The same pass can also return each vector's
// norm (a cache keeps its keys' norms for the TempCache cosine search).
// Several token sets (e.g. a step's queries and current keys) can share one
// launch.
#include "common.hpp"
#include "launch.hpp"

namespace fastar {

// Up to kHashBatch token sets hashed with the same planes in one launch
// (grid z = set): one launch instead of one per set.
struct HashSets {
    const void* x[kHashBatch];
    int N[kHashBatch];
    uint16_t* ids[kHashBatch];
    float* norms[kHashBatch];
};

// One block of 4 waves hashes 64 * GPW vectors of one head and one token set
// (GPW 16-vector groups per wave; bf16 blocks take GPW = 2, so the planes are
// staged once per 128 vectors and every wave has two groups' loads in
// flight).  The projections X R^T run on the matrix cores: the P <= 16
// planes are the 16 rows of one MFMA block (rows past P are zero and their
// bits dropped) and 16 vectors its columns.  A lane ends with the projections
// of planes 4g..4g+3 (g = lane / 16) onto its vector, turns their signs into
// id bits, and the four lane groups OR their bits together.
//
// bf16 vectors: v_mfma_f32_16x16x32_bf16 takes the vectors' bits as loaded
// (lane group g supplies dimensions 32c + 8g .. 32c + 8g + 7 of k-step c, one
// 16-byte load, so a wave's load reads one contiguous 64-byte run of each of
// 16 vectors).  Each fp32 plane element is split exactly into three bf16
// terms, p = hi + mid + lo (truncations: hi keeps the top 8 significand bits,
// mid the next 8, lo the last 8), so every product is exact and the three
// projections, accumulated in fp32 and added smallest first, carry the error
// of one fp32 dot product.  Three bf16 MFMAs per 32 dimensions take a fifth of
// the issue time of fp32 MFMAs.
//
// fp32 vectors: v_mfma_f32_16x16x4f32 on the fp32 values, lane group g
// summing the same dimensions; two accumulator chains overlap.
template <typename T, int D, int GPW>
__global__ __launch_bounds__(256) void hash_kernel(const HashSets sets, const float* __restrict__ planes,
                                                   int P) {
    constexpr bool BF = sizeof(T) == 2;
    constexpr int VPB = 64 * GPW;
    constexpr int DG = D / 4;                  // dimensions per lane group
    constexpr int STR = D + 4;                 // fp32 LDS row stride (floats): distinct banks per quarter-wave
    constexpr int PSTR = D + 8;                // bf16 LDS row stride (elements): 16-byte pad
    __shared__ __align__(16) float pl[BF ? 4 : 16 * STR];
    __shared__ __align__(16) uint16_t pb[3][BF ? 16 * PSTR : 8];
    const T* __restrict__ x = static_cast<const T*>(sets.x[blockIdx.z]);
    const int N = sets.N[blockIdx.z];
    uint16_t* __restrict__ ids = sets.ids[blockIdx.z];
    float* __restrict__ norms = sets.norms[blockIdx.z];
    const int h = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    if (blockIdx.x * VPB >= N) return;         // block uniform
    // group q of wave w holds vectors i0 + 16q + c16
    const int i0 = blockIdx.x * VPB + w * 16 * GPW;

    f32x4 proj[GPW];
    float sq[GPW];
    if constexpr (BF) {
        constexpr int KS = D / 32;
        // every group's 8 dimensions of each k-step, issued before the planes
        u32x4 xr[GPW][KS];
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            const int i = i0 + 16 * q + c16;
            const T* row = x + (static_cast<size_t>(h) * N + (i < N ? i : 0)) * D + g * 8;
#pragma unroll
            for (int c = 0; c < KS; ++c) {
                xr[q][c] = u32x4{0u, 0u, 0u, 0u};
                if (i < N) xr[q][c] = *reinterpret_cast<const u32x4*>(row + 32 * c);
            }
        }
        // the head's planes as three exact bf16 parts, rows past P zero;
        // thread (r, k0) splits D / 16 consecutive elements of row r
        {
            constexpr int EPT = D / 16;
            const int r = tid >> 4, k0 = (tid & 15) * EPT;
            float pv[EPT];
#pragma unroll
            for (int e = 0; e < EPT; e += 4) {
                float4 v4 = make_float4(0.f, 0.f, 0.f, 0.f);
                if (r < P) v4 = *reinterpret_cast<const float4*>(planes + (static_cast<size_t>(h) * P + r) * D + k0 + e);
                pv[e] = v4.x; pv[e + 1] = v4.y; pv[e + 2] = v4.z; pv[e + 3] = v4.w;
            }
            uint32_t hw[EPT / 2], mw[EPT / 2], lw[EPT / 2];
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                const float v = pv[e];
                const uint32_t hi = __float_as_uint(v) & 0xFFFF0000u;
                const float r1 = v - __uint_as_float(hi);
                const uint32_t mid = __float_as_uint(r1) & 0xFFFF0000u;
                const uint32_t lo = __float_as_uint(r1 - __uint_as_float(mid)) & 0xFFFF0000u;
                const int sh = (e & 1) ? 0 : 16;            // element e -> half (e & 1) of word e / 2
                if ((e & 1) == 0) { hw[e / 2] = hi >> sh; mw[e / 2] = mid >> sh; lw[e / 2] = lo >> sh; }
                else { hw[e / 2] |= hi; mw[e / 2] |= mid; lw[e / 2] |= lo; }
            }
#pragma unroll
            for (int e = 0; e < EPT / 2; e += 2) {
                *reinterpret_cast<uint2*>(&pb[0][r * PSTR + k0 + 2 * e]) = make_uint2(hw[e], hw[e + 1]);
                *reinterpret_cast<uint2*>(&pb[1][r * PSTR + k0 + 2 * e]) = make_uint2(mw[e], mw[e + 1]);
                *reinterpret_cast<uint2*>(&pb[2][r * PSTR + k0 + 2 * e]) = make_uint2(lw[e], lw[e + 1]);
            }
        }
        __syncthreads();
        bf16x8_t a[3][KS];
#pragma unroll
        for (int part = 0; part < 3; ++part)
#pragma unroll
            for (int c = 0; c < KS; ++c)
                a[part][c] = *reinterpret_cast<const bf16x8_t*>(&pb[part][c16 * PSTR + 32 * c + 8 * g]);
#pragma unroll
        for (int q = 0; q < GPW; ++q) {
            f32x4 acc[3] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int c = 0; c < KS; ++c) {
                const bf16x8_t b = __builtin_bit_cast(bf16x8_t, xr[q][c]);
#pragma unroll
                for (int part = 0; part < 3; ++part)
                    acc[part] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[part][c], b, acc[part], 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) proj[q][r] = acc[0][r] + (acc[1][r] + acc[2][r]);
            sq[q] = 0.f;
            if (norms) {
#pragma unroll
                for (int c = 0; c < KS; ++c)
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float lo = __uint_as_float(xr[q][c][k] << 16);
                        const float hi = __uint_as_float(xr[q][c][k] & 0xFFFF0000u);
                        sq[q] = __builtin_fmaf(lo, lo, sq[q]);
                        sq[q] = __builtin_fmaf(hi, hi, sq[q]);
                    }
            }
        }
    } else {
        static_assert(GPW == 1, "fp32 blocks take one group per wave");
        const int i = i0 + c16;
        const T* row = x + (static_cast<size_t>(h) * N + (i < N ? i : 0)) * D + g * 8;
        // the head's planes, rows past P zero
        for (int k = tid; k < 16 * (D / 4); k += 256) {
            const int r = k / (D / 4), q = k % (D / 4);
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < P) v = *reinterpret_cast<const float4*>(planes + (static_cast<size_t>(h) * P + r) * D + 4 * q);
            *reinterpret_cast<float4*>(&pl[r * STR + 4 * q]) = v;
        }
        // this lane's slice of its vector: xv[8c + j] = x[32c + 8g + j]
        float xv[DG];
#pragma unroll
        for (int e = 0; e < DG; e += 8) {
            float v[8];
            load8_f32(row + 4 * e, v);
#pragma unroll
            for (int k = 0; k < 8; ++k) xv[e + k] = i < N ? v[k] : 0.f;
        }
        __syncthreads();
        // the plane element paired with xv[e]
        auto dim = [&](int e) { return (e >> 3) * 32 + g * 8 + (e & 7); };
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        const float* prow = &pl[c16 * STR];
#pragma unroll
        for (int e = 0; e < DG / 2; e += 4) {
            const float4 a = *reinterpret_cast<const float4*>(prow + dim(e));
            const float4 b = *reinterpret_cast<const float4*>(prow + dim(DG / 2 + e));
            acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, xv[e], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(b.x, xv[DG / 2 + e], acc1, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, xv[e + 1], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(b.y, xv[DG / 2 + e + 1], acc1, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, xv[e + 2], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(b.z, xv[DG / 2 + e + 2], acc1, 0, 0, 0);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, xv[e + 3], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(b.w, xv[DG / 2 + e + 3], acc1, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) proj[0][r] = acc0[r] + acc1[r];
        sq[0] = 0.f;
        if (norms) {
#pragma unroll
            for (int e = 0; e < DG; ++e) sq[0] = __builtin_fmaf(xv[e], xv[e], sq[0]);
        }
    }
#pragma unroll
    for (int q = 0; q < GPW; ++q) {
        uint32_t bits = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int pidx = 4 * g + r;
            if (pidx < P && proj[q][r] >= 0.f) bits |= 1u << pidx;
        }
        bits |= __shfl_xor(bits, 16);
        bits |= __shfl_xor(bits, 32);
        float s2 = sq[q];
        if (norms) {
            s2 += __shfl_xor(s2, 16);
            s2 += __shfl_xor(s2, 32);
        }
        const int i = i0 + 16 * q + c16;
        if (i < N && g == 0) {
            ids[static_cast<size_t>(h) * N + i] = static_cast<uint16_t>(bits);
            if (norms) norms[static_cast<size_t>(h) * N + i] = __builtin_sqrtf(s2);
        }
    }
}

// bf16 blocks take two 16-vector groups per wave (128 vectors per block;
// the step's three-set launch: 9.7 us against 12.0 with four groups and 12.6
// with one), fp32 blocks one.
template <typename T, int D>
static hipError_t hash_dispatch_p(const HashSets& sets, int count, int H, const float* planes, int P,
                                  hipStream_t s) {
    constexpr int GPW = sizeof(T) == 2 ? 2 : 1;
    int nmax = 0;
    for (int i = 0; i < count; ++i) nmax = sets.N[i] > nmax ? sets.N[i] : nmax;
    timer_begin("ann_hash", s);
    hipLaunchKernelGGL((hash_kernel<T, D, GPW>), dim3((nmax + 64 * GPW - 1) / (64 * GPW), H, count), dim3(256), 0,
                       s, sets, planes, P);
    timer_end(s);
    return hipGetLastError();
}

hipError_t launch_hash_batch(int count, const void* const* x, const int* N, uint16_t* const* ids,
                             float* const* norms, bool bf16, int H, int d, const float* planes, int P,
                             hipStream_t s) {
    HashSets sets;
    int used = 0;
    for (int i = 0; i < count && i < kHashBatch; ++i) {
        if (N[i] == 0) continue;
        sets.x[used] = x[i];
        sets.N[used] = N[i];
        sets.ids[used] = ids[i];
        sets.norms[used] = norms ? norms[i] : nullptr;
        ++used;
    }
    if (used == 0 || H == 0) return hipSuccess;
    for (int i = used; i < kHashBatch; ++i) {
        sets.x[i] = nullptr;
        sets.N[i] = 0;
        sets.ids[i] = nullptr;
        sets.norms[i] = nullptr;
    }
    if (bf16)
        return d == 64 ? hash_dispatch_p<uint16_t, 64>(sets, used, H, planes, P, s)
                       : hash_dispatch_p<uint16_t, 128>(sets, used, H, planes, P, s);
    return d == 64 ? hash_dispatch_p<float, 64>(sets, used, H, planes, P, s)
                   : hash_dispatch_p<float, 128>(sets, used, H, planes, P, s);
}

hipError_t launch_hash(const void* x, bool bf16, int H, int N, int d, const float* planes, int P,
                       uint16_t* ids, float* norms, hipStream_t s) {
    return launch_hash_batch(1, &x, &N, &ids, &norms, bf16, H, d, planes, P, s);
}

}  // namespace fastar
