// Host-side interface of the fused attention kernel (internal to libtpshard).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tps {
// qkv: bf16 [b*s, 3*Hl*d] ([Q heads | K heads | V heads] per token);
// O: bf16 [b*s, Hl*d]. d in {64, 128}.
hipError_t attn_fwd(const uint16_t* qkv, uint16_t* O, int b, int s, int Hl, int d, bool causal, hipStream_t st);
}  // namespace tps
