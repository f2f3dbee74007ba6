// kda_chunk.hip -- shape dispatch of the chunk engine (kda_engine.h), whose
// instantiations live in one translation unit per shape family
// (kda_chunk_*.hip).

#include "kda_internal.h"

namespace kda {

hipError_t launch_engine_bf16_128x128(int mode, int dv, int nb, const EngineArgs &a, hipStream_t s);
hipError_t launch_engine_bf16_64x128(int mode, int dv, int nb, const EngineArgs &a, hipStream_t s);
hipError_t launch_engine_bf16_128x64(int mode, int dv, int nb, const EngineArgs &a, hipStream_t s);
hipError_t launch_engine_bf16_64x64(int mode, int dv, int nb, const EngineArgs &a, hipStream_t s);
hipError_t launch_engine_f32_64(int mode, int dv, int nb, const EngineArgs &a, hipStream_t s);

bool engine_supported(bool bf16, int dk, int dv, int nb) {
    const bool dims = (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
    if (bf16) return dims && (nb == 64 || (nb == 128 && dv == 128));
    // fp32 operands: dk = 128 (whose hand-off tiles do not fit in LDS) runs
    // the token-recurrent kernel
    return dims && nb == 64;
}

int engine_pick_nb(bool bf16, int dk, int dv, int64_t units, int mode) {
    (void)dk;
    (void)mode;
    if (!bf16 || dv == 64) return 64;
    // Split the value columns when the grid would leave most CUs idle.
    return units >= 256 ? 128 : 64;
}

hipError_t launch_engine(int mode, bool bf16, int dk, int dv, int nb, const EngineArgs &a,
                         hipStream_t s) {
    if (!engine_supported(bf16, dk, dv, nb)) return hipErrorInvalidValue;
    if (recurrent_supported(bf16, dk, dv)) return launch_recurrent(mode, dk, dv, a, s);
    if (!bf16) return launch_engine_f32_64(mode, dv, nb, a, s);
    if (dk == 128) return dv == 128 ? launch_engine_bf16_128x128(mode, dv, nb, a, s)
                                    : launch_engine_bf16_128x64(mode, dv, nb, a, s);
    return dv == 128 ? launch_engine_bf16_64x128(mode, dv, nb, a, s)
                     : launch_engine_bf16_64x64(mode, dv, nb, a, s);
}

}  // namespace kda
