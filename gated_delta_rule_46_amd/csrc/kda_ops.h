// Internal interfaces of the decode step (kda_decode.hip) and the short
// convolution (kda_conv.hip) with the C ABI (kda_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {

// One-token step against a state pool (kda_decode.hip).
struct DecodeArgs {
    const void *q, *k, *v;       // [N,H,dk] / [N,H,dv], io dtype
    const float *g, *beta;       // [N,H,dk], [N,H]: gates or, with gate_logits, logits
    void *o;                     // [N,H,dv]
    float *pool;                 // [n_slots,H,dk,dv]
    int64_t n_slots;
    const int32_t *read_idx, *write_idx;   // [N]
    int32_t N, H;
    float scale;
    int32_t l2norm;
    int32_t gate_logits;
};
bool decode_supported(int dk, int dv);
hipError_t launch_decode(bool bf16, int dk, int dv, const DecodeArgs &a, hipStream_t s);

// Short causal convolution over tokens (kda_conv.hip).
struct ConvArgs {
    const void *x;               // [T, C] I/O dtype
    void *y;                     // [T, C] I/O dtype
    void *win;                   // window slots [n_slots, W-1, C], I/O dtype (nullable)
    const float *weight;         // [C, W]
    const float *bias;           // [C] (nullable)
    const int64_t *cu;           // [N+1] sequence (or segment) bounds
    int32_t N, C;
    int64_t T, n_slots;
    const int32_t *read_idx, *write_idx;   // [N] (nullable)
    int32_t act;                 // 0 none, 1 SiLU
};
hipError_t launch_conv(bool bf16, int width, const ConvArgs &a, hipStream_t s);
hipError_t launch_conv_halo(bool bf16, int width, const ConvArgs &a, hipStream_t s);

}  // namespace kda
