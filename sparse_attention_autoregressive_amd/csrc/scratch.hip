// AnnSA on a static scratch array, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation).  The array is a file-scope device variable: every
// device the library's code is loaded on holds its own copy at its own
// address.  Host code never passes the array's name to a kernel (on the host
// that name is only a stand-in for the device symbol); the device address is
// resolved with hipGetSymbolAddress once per device, with that device
// current, and only that address reaches the kernels, as the workspace of the
// ordinary AnnSA sequence.
#include <hip/hip_runtime.h>

#include <mutex>

#include "annsa_entry.hpp"
#include "fastar.h"

namespace {

constexpr size_t kScratchBytes = FASTAR_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};     // the array's address on each device, once resolved

// The array's device address on the calling thread's current device.
fastar_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FASTAR_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FASTAR_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FASTAR_OK;
}

}  // namespace

extern "C" fastar_status fastar_annsa_forward_static(const void* q, const uint16_t* q_ids, int32_t H,
                                                     int32_t Nq, int32_t d, int32_t dtype,
                                                     const fastar_cache* cache, const void* k_cur,
                                                     const void* v_cur, const uint16_t* kcur_ids,
                                                     int32_t Ncur, int32_t P, float scale, void* out,
                                                     int32_t out_dtype, float* lse, int32_t* best,
                                                     float* best_cos, void* stream) {
    size_t need = 0;
    const fastar_status vs = fastar::annsa_validate(q, q_ids, H, Nq, d, dtype, cache, k_cur, v_cur,
                                                    kcur_ids, Ncur, P, 1, scale, out, out_dtype, best,
                                                    best_cos, &need);
    if (vs != FASTAR_OK) return vs;
    if (need > kScratchBytes) return FASTAR_ESCRATCH;
    if (static_cast<long long>(H) * Nq == 0) return FASTAR_OK;
    void* ws = nullptr;
    const fastar_status as = scratch_address(&ws);
    if (as != FASTAR_OK) return as;
    return fastar::annsa_impl(q, q_ids, H, Nq, d, dtype, cache, k_cur, v_cur, kcur_ids, Ncur, P, 1, scale,
                              out, out_dtype, lse, best, best_cos, ws, kScratchBytes, stream);
}
