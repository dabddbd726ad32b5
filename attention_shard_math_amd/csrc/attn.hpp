// Host-side interface of the fused attention kernel (internal to libtpshard).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tps {
// qkv: bf16 [b*s, 3*Hl*d] ([Q heads | K heads | V heads] per token);
// O: bf16 [b*s, Hl*d]. d in {64, 128}. lse (nullable): float32 [b, Hl, s], the
// natural-log log-sum-exp of each query's scaled scores.
hipError_t attn_fwd(const uint16_t* qkv, uint16_t* O, int b, int s, int Hl, int d, bool causal, hipStream_t st,
                    float* lse = nullptr);

// Backward of attn_fwd over the same layout: dQKV bf16 [b*s, 3*Hl*d] from qkv, O,
// dO bf16 [b*s, Hl*d] and lse. ws: attn_bwd_workspace(b, s, Hl, d) bytes of
// scratch (rowsum(dO*O) and the fp32 partials of split walks).
size_t attn_bwd_workspace(int b, int s, int Hl, int d);
hipError_t attn_bwd(const uint16_t* qkv, const uint16_t* O, const uint16_t* dO, const float* lse, uint16_t* dqkv,
                    void* ws, int b, int s, int Hl, int d, bool causal, hipStream_t st);
}  // namespace tps
