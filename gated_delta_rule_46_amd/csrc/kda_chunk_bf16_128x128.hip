// kda_chunk_bf16_128x128.hip -- the chunk engine instantiated for bf16, dk = dv = 128.

#include "kda_engine.h"

namespace kda {

hipError_t launch_engine_bf16_128x128(int mode, int dv, int nb, const EngineArgs &a, hipStream_t s) {
    if (dv == 128 && nb == 128) return launch_modes<128, 128, 128, true>(mode, a, s);
    if (dv == 128 && nb == 64) return launch_modes<128, 128, 64, true>(mode, a, s);
    return hipErrorInvalidValue;
}

}  // namespace kda
