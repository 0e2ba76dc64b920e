// AnnSA's host sequence, shared by the workspace entry point and the
// static-scratch entry point (both defined with the C ABI).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "fastar.h"

namespace fastar {

// Host-side validation of an AnnSA call (every rule of fastar_annsa_forward
// and fastar_annsa_multi_forward); on success ``*need`` is the workspace the
// call takes, in bytes.  Touches no device state.
fastar_status annsa_validate(const void* q, const uint16_t* q_ids, int32_t H, int32_t Nq, int32_t d,
                             int32_t dtype, const fastar_cache* cache, const void* k_cur,
                             const void* v_cur, const uint16_t* kcur_ids, int32_t Ncur, int32_t P,
                             int32_t tables, float scale, const void* out, int32_t out_dtype,
                             const int32_t* best, const float* best_cos, size_t* need);

// Validates, then enqueues the bucket sort and the attention launch of each
// table on ``stream`` with ``ws`` (ws_bytes long) as the workspace.
fastar_status annsa_impl(const void* q, const uint16_t* q_ids, int32_t H, int32_t Nq, int32_t d,
                         int32_t dtype, const fastar_cache* cache, const void* k_cur, const void* v_cur,
                         const uint16_t* kcur_ids, int32_t Ncur, int32_t P, int32_t tables, float scale,
                         void* out, int32_t out_dtype, float* lse, int32_t* best, float* best_cos,
                         void* ws, size_t ws_bytes, void* stream);

}  // namespace fastar
