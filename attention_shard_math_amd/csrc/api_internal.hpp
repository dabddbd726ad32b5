// Internal interface shared by the C-ABI translation units of libtpshard (not exported).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tpshard.h"

namespace tps {

// Sets the calling thread's tp_last_error() text and returns st.
tp_status api_fail(tp_status st, const char* fmt, ...);
// Clears the calling thread's tp_last_error() text and returns TP_OK.
tp_status api_ok();

// Host checks of the MLP backward's sizes and tensor pointers (not the workspace).
tp_status mlp_bwd_validate(const char* fn, int64_t M, int64_t h, int64_t f, const void* X, const void* A_i,
                           const void* B_i, const void* U_i, const void* Y_i, const void* dZ, const float* dX_i,
                           const float* dA_i, const float* dB_i);

// The four products of the MLP backward (dU, dB, dA, dX) on stream s, with dU a bf16
// [M, f] scratch buffer and sk the stream-K area (nullable: no product runs stream-K).
tp_status mlp_bwd_products(const char* fn, int64_t M, int64_t h, int64_t f, const void* X, const void* A_i,
                           const void* B_i, const void* U_i, const void* Y_i, const void* dZ, float* dX_i,
                           float* dA_i, float* dB_i, uint16_t* dU, void* sk, hipStream_t s);

}  // namespace tps
