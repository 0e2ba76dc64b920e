// Random-hyperplane bucket ids (the LSH that places queries, cache keys,
// current keys and prompt keys in one shared bucket space; FAST-AR summary,
// "2. Core Components", parts A and B):
//
//   id(x) = sum_p [<x, r_p> >= 0] << p
//
// The projections onto the P <= 16 planes are one 16-row matrix-core block per
// 16 vectors (see hash_kernel).  The same pass can also return each vector's
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

// One block of 4 waves hashes 64 vectors of one head and one token set.  The
// projections X R^T run on the matrix cores (fp32 v_mfma_f32_16x16x4f32; bf16
// inputs widen exactly, the planes stay fp32): the P <= 16 planes are the 16
// rows of one MFMA block (rows past P are zero and their bits dropped), the
// wave's 16 vectors its columns, and lane group g sums dimensions g*D/4 ..
// (g+1)*D/4-1 of both operands, so each lane reads contiguous runs.  A lane
// then holds the projections of planes 4g..4g+3 onto its vector and turns
// their signs into id bits; the four groups OR their bits together.  Two
// accumulator chains (the two halves of each group's dimensions) overlap.
template <typename T, int D>
__global__ __launch_bounds__(256) void hash_kernel(const HashSets sets, const float* __restrict__ planes,
                                                   int P) {
    constexpr int DG = D / 4;                  // dimensions per lane group
    constexpr int STR = D + 4;                 // LDS row stride (floats): distinct banks per quarter-wave
    __shared__ __align__(16) float pl[16 * STR];
    const T* __restrict__ x = static_cast<const T*>(sets.x[blockIdx.z]);
    const int N = sets.N[blockIdx.z];
    uint16_t* __restrict__ ids = sets.ids[blockIdx.z];
    float* __restrict__ norms = sets.norms[blockIdx.z];
    const int h = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int i = blockIdx.x * 64 + w * 16 + c16;
    if (blockIdx.x * 64 >= N) return;          // block uniform

    // the head's planes, rows past P zero
    for (int k = tid; k < 16 * (D / 4); k += 256) {
        const int r = k / (D / 4), q = k % (D / 4);
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r < P) v = *reinterpret_cast<const float4*>(planes + (static_cast<size_t>(h) * P + r) * D + 4 * q);
        *reinterpret_cast<float4*>(&pl[r * STR + 4 * q]) = v;
    }
    // this lane's slice of its vector
    const bool valid = i < N;
    float xv[DG];
    {
        const T* row = x + (static_cast<size_t>(h) * N + (valid ? i : 0)) * D + g * DG;
#pragma unroll
        for (int e = 0; e < DG; e += 8) {
            float v[8];
            load8_f32(row + e, v);
#pragma unroll
            for (int k = 0; k < 8; ++k) xv[e + k] = valid ? v[k] : 0.f;
        }
    }
    __syncthreads();

    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    const float* prow = &pl[c16 * STR + g * DG];
#pragma unroll
    for (int e = 0; e < DG / 2; e += 4) {
        const float4 a = *reinterpret_cast<const float4*>(prow + e);
        const float4 b = *reinterpret_cast<const float4*>(prow + DG / 2 + e);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, xv[e], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(b.x, xv[DG / 2 + e], acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, xv[e + 1], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(b.y, xv[DG / 2 + e + 1], acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, xv[e + 2], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(b.z, xv[DG / 2 + e + 2], acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, xv[e + 3], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(b.w, xv[DG / 2 + e + 3], acc1, 0, 0, 0);
    }
    uint32_t bits = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int pidx = 4 * g + r;
        if (pidx < P && acc0[r] + acc1[r] >= 0.f) bits |= 1u << pidx;
    }
    bits |= __shfl_xor(bits, 16);
    bits |= __shfl_xor(bits, 32);
    float sq = 0.f;
    if (norms) {
#pragma unroll
        for (int e = 0; e < DG; ++e) sq = __builtin_fmaf(xv[e], xv[e], sq);
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
    }
    if (valid && g == 0) {
        ids[static_cast<size_t>(h) * N + i] = static_cast<uint16_t>(bits);
        if (norms) norms[static_cast<size_t>(h) * N + i] = __builtin_sqrtf(sq);
    }
}

template <typename T, int D>
static hipError_t hash_dispatch_p(const HashSets& sets, int count, int H, const float* planes, int P,
                                  hipStream_t s) {
    int nmax = 0;
    for (int i = 0; i < count; ++i) nmax = sets.N[i] > nmax ? sets.N[i] : nmax;
    dim3 grid((nmax + 63) / 64, H, count);
    timer_begin("ann_hash", s);
    hipLaunchKernelGGL((hash_kernel<T, D>), grid, dim3(256), 0, s, sets, planes, P);
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
