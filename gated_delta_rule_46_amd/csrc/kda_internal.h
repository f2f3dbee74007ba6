// Internal interfaces between the C ABI (kda_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kChunk = 64;

// Bit patterns by value.  __builtin_bit_cast whose operand is an element of an
// ext_vector_type vector (v[i]) reads element 0 whatever i is (hipcc of
// ROCm 7.2), so every bit-level test or reinterpretation of a single element
// goes through these helpers, whose parameter is a value.
__device__ __forceinline__ uint32_t f32_bits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bits_f32(uint32_t x) { return __builtin_bit_cast(float, x); }

// Returns x unchanged, but hides its value from the optimiser.  Lane indices
// are laundered through it at the top of a phase or a product so that the
// addresses and masks derived from them are recomputed there instead of being
// hoisted out of the loops around it (hundreds of hoisted values otherwise
// exhaust the register file).
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Prefill: sequences from S0.  Package: value blocks of every segment from a
// zero state (o_local, D, sub_D).  PackageM: the segment's linear part M (and
// sub_M) from the identity.  Fixup: outputs corrected from S_in.  PackageVM:
// value blocks and M blocks in one launch, the M blocks dispatched last.
// FixOp: the fix-up of the units a fix-up operator covers (fixop_kernel).
enum EngineMode : int {
    kModePrefill = 0, kModePackage = 1, kModeFixup = 2, kModePackageM = 3, kModePackageVM = 4,
    kModeFixOp = 5
};

// Arguments of the fused chunk engine (one workgroup per (unit, head,
// column block); a unit is a sequence for prefill and a segment otherwise).
struct EngineArgs {
    const void *q, *k, *v;       // [T,H,dk] / [T,H,dv], io dtype
    const float *g, *beta;       // [T,H,dk], [T,H]
    void *o;                     // [T,H,dv]: written (prefill/package) or updated (fixup)
    const int64_t *bounds;       // [n_units+1] token offsets (cu_seqlens or seg_start)
    const int32_t *order;        // [n_units] longest-first unit order, NULL = identity
    int32_t n_units;
    int32_t H;
    int32_t ncb;                 // column blocks of the launch (dv / NB, or dk / NB for M)
    int32_t ncb_m;               // PackageVM: column blocks of the M part (dk / min(NB, dk))
    const float *S_init;         // prefill: S0 (nullable); fixup: S_in
    float *S_out;                // prefill: S_final (nullable); package: D
    float *M_out;                // package: M
    int32_t interval;            // checkpoint interval in tokens, 0 = none
    const int64_t *ckpt_off;     // prefill: first rung row per sequence (nullable)
    float *ckpt_S;               // prefill: checkpoint states; package: sub_D; fixup: rung
                                 //   states written beside the outputs (nullable)
    const float *ckpt_in;        // fixup with rungs: sub_D of every rung (read)
    float *ckpt_M;               // package: sub_M (nullable)
    float scale;
    int32_t l2norm;
    // Prefill from a state pool (all nullable): the initial state of unit u is
    // slot s_in_idx[u] of S_init and its final state goes to slot s_out_idx[u]
    // of S_out (slots outside [0, n_slots): zero state / not stored); pos0[u]
    // is the absolute position of the unit's first token, which places the
    // checkpoint rungs on the original sequence's grid.
    const int32_t *s_in_idx, *s_out_idx;
    int64_t n_slots;
    const int64_t *pos0;
    // Fix-up operator (nullable).  Package: the M blocks write, for the first
    // X_chunks chunks of unit u, X[u][t - t0][h] = their outputs (the
    // identity's map to output t) and X_len[u][h][b] = the chunks after which
    // columns 64b..64b+63 of the propagated identity are exactly zero (-1:
    // not within X_chunks).  Fix-up: units whose X_len are all >= 0 are
    // corrected from X instead of the recurrence.
    void *X;                     // [n_units, X_chunks * 64, H, dk], io dtype
    int32_t *X_len;              // [n_units, H, dk / 64]
    int32_t X_chunks;
    // and the propagated identity at the first rung of X_interval after the
    // unit's start when it falls within the X_chunks chunks (nullable)
    float *X_Pi;                 // [n_units, H, dk, dk]
    int32_t X_interval;
    // package of split segments: X_per sub-segments per segment, the operator
    // of segment u / X_per written by its first sub-segment (0 or 1: none split)
    int32_t X_per;
    // and, of the later sub-segments (u % X_per != 0), each sub-segment's own
    // operator (nullable: none), in slot (u % X_per - 1) * (n_units / X_per) +
    // u / X_per: it corrects the sub-segment's rows from the state that the
    // sub-segments before it accumulated.  Its counts are valid at the
    // sub-segment's end without vanishing.
    void *Xs;                    // [X_per - 1, n_units / X_per, Xs_chunks * 64, H, dk]
    int32_t *Xs_len;             // [X_per - 1, n_units / X_per, H, dk / 64]
    float *Xs_Pi;                // [X_per - 1, n_units / X_per, H, dk, dk] (nullable)
    int32_t Xs_chunks;
    int32_t Xs_interval;
    // Package of split segments: the last sub-segment of segment j (u % X_per
    // == X_per - 1) writes its D and M into slot j of S_last and M_last, where
    // the merge composes them in place (nullable: slot u of S_out / M_out).
    float *S_last, *M_last;
    // FixOp writes the route of every unit (1: the recurrence), the fix-up
    // launch after it skips the units with route 0 (nullable: none skipped).
    // FixOp reads X, X_len and X_Pi at the unit's position in `order` and the
    // incoming state and the route at the unit itself.
    int32_t *X_route;            // [n_units, H]
};

// Slot of a package output (`size` floats per head) of unit u: slot u of
// base, or slot u / per of last for the last sub-segment of a split segment.
__device__ __forceinline__ float *package_slot(float *base, float *last, int per, int u, int H,
                                               int h, int64_t size) {
    if (last && per > 1 && u % per == per - 1) return last + ((int64_t)(u / per) * H + h) * size;
    return base + ((int64_t)u * H + h) * size;
}

// Launches the engine.  bf16 selects bf16 I/O (bf16 MFMA operands) versus
// fp32 I/O (fp32 MFMA).  nb is the value-column block width.  Returns a HIP
// error code.  `grid_units` is n_units (the launch covers every unit).
hipError_t launch_engine(int mode, bool bf16, int dk, int dv, int nb, const EngineArgs &a,
                         hipStream_t stream);
// Token-recurrent kernel for the shapes whose fp32 hand-off tiles do not fit
// the chunk engine's LDS (fp32 I/O, dk = 128); same modes and arguments, with
// a.ncb = dv / 64 and a.ncb_m = dk / 64 (kda_recurrent.hip).
bool recurrent_supported(bool bf16, int dk, int dv);
hipError_t launch_recurrent(int mode, int dk, int dv, const EngineArgs &a, hipStream_t stream);
bool engine_supported(bool bf16, int dk, int dv, int nb);
int engine_pick_nb(bool bf16, int dk, int dv, int64_t units, int mode);

// Longest-first schedule of n sequences from cu_seqlens (device), into order[n].
hipError_t launch_plan(const int64_t *cu_seqlens, int32_t n, int32_t *order, hipStream_t s);

// Package scans (fp32).
// flags (nullable): sequential_workspace(H, nseg) bytes, where a first launch
// tests every M once for the scan.
size_t sequential_workspace(int H, int nseg);
hipError_t launch_scan_sequential(int dk, int dv, int H, int nseg, const float *M,
                                  const float *D, const float *S0, float *S_in,
                                  float *S_final, int *flags, hipStream_t s);
hipError_t launch_scan_blelloch(int dk, int dv, int H, int nseg, const float *M,
                                const float *D, const float *S0, float *S_in,
                                float *S_final, void *ws, hipStream_t s);
size_t blelloch_workspace(int dk, int dv, int H, int nseg);
int blelloch_max_segments();   // largest nseg the Blelloch scan takes

// bounds[j] = min(j*L, T) for j = 0..nseg (device int64).
hipError_t launch_even_bounds(int64_t *bounds, int nseg, int64_t L, int64_t T, hipStream_t s);

// Segments split into f sub-segments (kda_segment_package): bounds and merge
// orders, the in-place composition of step k, and the sub_M rungs of step k.
hipError_t launch_split_bounds(const int64_t *seg_start, int nseg, int f, int64_t *sb,
                               int32_t *ord, hipStream_t s);
hipError_t launch_split_compose(int dk, int dv, int H, int nseg, int f, int k, float *Ms,
                                float *Ds, float *M_out, float *D_out, hipStream_t s);
hipError_t launch_split_rung_m(int dk, int H, int nseg, int f, int k, const int64_t *sb,
                               int interval, int64_t rows, const float *Ms, float *sub_M,
                               hipStream_t s);

// Debug check of device-side inputs into report[0..fields) (kda_validate.hip).
hipError_t launch_validate(int64_t T, int H, int dk, const int64_t *bounds, int n, int aligned,
                           const float *g, const float *beta, int *report, int fields,
                           hipStream_t s);

// Segment-path checkpoints: states[row] = sub_M[row] S_in[j] + sub_D[row].
hipError_t launch_ckpt_write(int dk, int dv, int H, int64_t T, const int64_t *seg_start,
                             int nseg, int interval, const float *S_in, const float *sub_M,
                             const float *sub_D, float *states, hipStream_t s);

}  // namespace kda
