// AnnCA prompt selection (FAST-AR blog, "2. AnnCA"; summary, "2. Core
// Components" B): for each (head, frame), the buckets occupied by the frame's
// queries form a bitmap in LDS; a prompt token is kept iff its bucket bit is
// set.  Kept indices are compacted in ascending order with a block-wide
// ballot/scan, so the list (and the attention over it) is deterministic.
#include "common.hpp"
#include "launch.hpp"

namespace fastar {

__global__ __launch_bounds__(256) void annca_select_kernel(
    const uint16_t* __restrict__ q_ids, const uint16_t* __restrict__ kp_ids, int Nq, int frame_len,
    int L, int B, int32_t* __restrict__ idx, int32_t* __restrict__ cnt, uint8_t* __restrict__ keep,
    int32_t* __restrict__ keep_count) {
    __shared__ uint32_t bits[32];
    __shared__ int smem[4];
    const int f = blockIdx.x, h = blockIdx.y, F = gridDim.x;
    if (threadIdx.x < 32) bits[threadIdx.x] = 0;
    __syncthreads();
    const uint16_t* qi = q_ids + static_cast<size_t>(h) * Nq + static_cast<size_t>(f) * frame_len;
    for (int i = threadIdx.x; i < frame_len; i += 256) {
        const int id = qi[i] & (B - 1);
        atomicOr(&bits[id >> 5], 1u << (id & 31));
    }
    __syncthreads();
    const uint16_t* pi = kp_ids + static_cast<size_t>(h) * L;
    const size_t row = static_cast<size_t>(h) * F + f;
    int carry = 0;
    for (int t0 = 0; t0 < L; t0 += 256) {
        const int t = t0 + threadIdx.x;
        int k = 0;
        if (t < L) {
            const int id = pi[t] & (B - 1);
            k = (bits[id >> 5] >> (id & 31)) & 1;
        }
        int total;
        const int pos = block_exclusive_scan<256>(k, smem, total);
        if (k) idx[row * L + carry + pos] = t;
        if (keep && t < L) keep[row * L + t] = static_cast<uint8_t>(k);
        carry += total;
    }
    if (threadIdx.x == 0) {
        cnt[row] = carry;
        if (keep_count) keep_count[row] = carry;
    }
}

hipError_t launch_annca_select(const uint16_t* q_ids, const uint16_t* kp_ids, int H, int Nq,
                               int frame_len, int L, int P, int32_t* idx, int32_t* cnt,
                               uint8_t* keep, int32_t* keep_count, hipStream_t s) {
    const int F = Nq / frame_len;
    if (H == 0 || F == 0) return hipSuccess;
    timer_begin("annca_select", s);
    hipLaunchKernelGGL(annca_select_kernel, dim3(F, H), dim3(256), 0, s, q_ids, kp_ids, Nq,
                       frame_len, L, 1 << P, idx, cnt, keep, keep_count);
    timer_end(s);
    return hipGetLastError();
}

}  // namespace fastar
