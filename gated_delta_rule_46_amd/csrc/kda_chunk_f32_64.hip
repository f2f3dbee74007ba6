// kda_chunk_f32_64.hip -- the chunk engine instantiated for fp32, dk = 64, dv in {64, 128}.

#include "kda_engine.h"

namespace kda {

hipError_t launch_engine_f32_64(int mode, int dv, int nb, const EngineArgs &a, hipStream_t s) {
    if (dv == 64 && nb == 64) return launch_modes<64, 64, 64, false>(mode, a, s);
    if (dv == 128 && nb == 64) return launch_modes<64, 128, 64, false>(mode, a, s);
    return hipErrorInvalidValue;
}

}  // namespace kda
