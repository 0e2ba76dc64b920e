// Random-hyperplane bucket ids (the LSH that places queries, cache keys,
// current keys and prompt keys in one shared bucket space; FAST-AR summary,
// "2. Core Components", parts A and B).
//
// HBM-bound: every element of x is read once.  Each group of d/8 lanes owns one
// vector; lane ``seg`` always handles the same 8 coordinates, so its slice of
// every hyperplane lives in registers for the whole kernel (staged once per
// block through LDS; no LDS traffic per element).  Partial projections are summed across the group with DPP row
// butterflies, which leave the same fp32 sum in every lane of the group.  The
// same pass can also return each vector's norm (a cache keeps its keys'
// norms for the TempCache cosine search).  Several token sets (e.g. a step's
// queries and current keys) can share one launch.
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

template <typename T, int D, int MAXP>
__global__ __launch_bounds__(256) void hash_kernel(const HashSets sets,
                                                   const float* __restrict__ planes, int P) {
    const T* __restrict__ x = static_cast<const T*>(sets.x[blockIdx.z]);
    const int N = sets.N[blockIdx.z];
    uint16_t* __restrict__ ids = sets.ids[blockIdx.z];
    float* __restrict__ norms = sets.norms[blockIdx.z];
    constexpr int LPV = D / 8;         // lanes per vector
    constexpr int VPB = 256 / LPV;     // vectors per block per step
    constexpr int UNROLL = 4;
    const int h = blockIdx.y;
    const int seg = threadIdx.x % LPV;
    const int vslot = threadIdx.x / LPV;

    // the head's planes go through LDS once per block (each block would
    // otherwise read them from L2 once per vector slot)
    __shared__ __align__(16) float spl[MAXP * D];
    for (int i = threadIdx.x; i < P * D / 4; i += 256)
        *reinterpret_cast<float4*>(&spl[4 * i]) =
            *reinterpret_cast<const float4*>(planes + static_cast<size_t>(h) * P * D + 4 * i);
    __syncthreads();
    float pl[MAXP][8];
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
        if (p < P) {
            const float4 a = *reinterpret_cast<const float4*>(&spl[p * D + seg * 8]);
            const float4 b = *reinterpret_cast<const float4*>(&spl[p * D + seg * 8 + 4]);
            pl[p][0] = a.x; pl[p][1] = a.y; pl[p][2] = a.z; pl[p][3] = a.w;
            pl[p][4] = b.x; pl[p][5] = b.y; pl[p][6] = b.z; pl[p][7] = b.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) pl[p][e] = 0.f;
        }
    }

    const T* xh = x + static_cast<size_t>(h) * N * D;
    uint16_t* idh = ids + static_cast<size_t>(h) * N;
    for (int base = blockIdx.x * VPB * UNROLL; base < N; base += gridDim.x * VPB * UNROLL) {
        float v[UNROLL][8];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int i = base + u * VPB + vslot;
            if (i < N) {
                load8_f32(xh + static_cast<size_t>(i) * D + seg * 8, v[u]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[u][e] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int i = base + u * VPB + vslot;
            uint32_t id = 0;
#pragma unroll
            for (int p = 0; p < MAXP; ++p) {
                if (p < P) {
                    float s = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) s = __builtin_fmaf(v[u][e], pl[p][e], s);
                    s = group_sum<(LPV < 16 ? LPV : 16)>(s);
                    id |= static_cast<uint32_t>(s >= 0.f) << p;
                }
            }
            if (seg == 0 && i < N) idh[i] = static_cast<uint16_t>(id);
            if (norms) {                                   // |x|, the cache keeps it per slot
                float sq = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) sq = __builtin_fmaf(v[u][e], v[u][e], sq);
                sq = group_sum<(LPV < 16 ? LPV : 16)>(sq);
                if (seg == 0 && i < N) norms[static_cast<size_t>(h) * N + i] = __builtin_sqrtf(sq);
            }
        }
    }
}

template <typename T, int D>
static hipError_t hash_dispatch_p(const HashSets& sets, int count, int H, const float* planes, int P,
                                  hipStream_t s) {
    constexpr int VPB = 256 / (D / 8);
    int nmax = 0;
    for (int i = 0; i < count; ++i) nmax = sets.N[i] > nmax ? sets.N[i] : nmax;
    int blocks = (nmax + VPB * 4 - 1) / (VPB * 4);
    if (blocks < 1) blocks = 1;
    dim3 grid(blocks, H, count);
    timer_begin("ann_hash", s);
    if (P <= 8)
        hipLaunchKernelGGL((hash_kernel<T, D, 8>), grid, dim3(256), 0, s, sets, planes, P);
    else
        hipLaunchKernelGGL((hash_kernel<T, D, 16>), grid, dim3(256), 0, s, sets, planes, P);
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
