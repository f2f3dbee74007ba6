// kda_chunk_bf16_128x64.hip -- the chunk engine instantiated for bf16, dk = 128, dv = 64.

#include "kda_engine.h"

namespace kda {

hipError_t launch_engine_bf16_128x64(int mode, int dv, int nb, const EngineArgs &a, hipStream_t s) {
    if (dv == 64 && nb == 64) return launch_modes<128, 64, 64, true>(mode, a, s);
    return hipErrorInvalidValue;
}

}  // namespace kda
