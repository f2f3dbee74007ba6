// kda_recurrent.hip -- token-recurrent KDA kernel for fp32 I/O with dk = 128.
//
// The chunk engine keeps its fp32 hand-off tiles in LDS; with a 128-wide key
// they need about 220 KiB against the 160 KiB a workgroup has, so this shape
// runs the recurrence one token at a time instead, in every mode the engine
// has (prefill from dense or pooled states with rungs, package value and M
// blocks, fix-up with rungs and the exact early exit).
//
// One wave per (unit, head, block of 64 state columns).  Lane j owns column
// cbase + j of the state for all DK rows, in registers, so every reduction of
// the token step runs inside the lane:
//     S <- Diag(alpha_t) S;   r = S^T k_t;   S <- S + k_t (beta_t (v_t - r))^T;
//     o_t = S^T q_t
// with k_t, q_t L2-normalised (x / sqrt(|x|^2 + 1e-6), q times scale) and
// alpha_t = exp(g_t).  The wave normalises k_t and q_t and forms alpha_t
// cooperatively (two channels per lane) and passes them to every lane through
// LDS.  The M blocks run the value-free form (v = 0) from the identity.

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kCols = 64;   // state columns per wave

template <int DK, int DV, int MODE, bool MB>
__device__ void recurrent_body(const EngineArgs &a, const int u, const int h, const int cbase,
                               const int64_t t0, const int64_t t1) {
    __shared__ float s_k[DK], s_q[DK], s_a[DK];
    static_assert(DK == 128, "two channels per lane");
    constexpr bool HAS_V = (MODE != kModeFixup) && !MB;
    constexpr bool HAS_O = !MB;
    constexpr bool CHECK0 = (MODE == kModeFixup) || MB;
    const int lane = threadIdx.x;
    const int H = a.H;
    constexpr int ldst = MB ? DK : DV;   // row length of the state this wave holds
    const int col = cbase + lane;
    const int64_t len = t1 - t0;
    float S[DK];
    // initial state
    {
        const float *src = nullptr;
        if (MODE == kModePrefill && a.s_in_idx) {
            const int32_t slot = a.s_in_idx[u];
            if (slot >= 0 && slot < a.n_slots) src = a.S_init + ((int64_t)slot * H + h) * DK * DV;
        } else if (MODE == kModePrefill && a.S_init) {
            src = a.S_init + ((int64_t)u * H + h) * DK * DV;
        }
        if (MODE == kModeFixup) src = a.S_init + ((int64_t)u * H + h) * DK * DV;
#pragma unroll
        for (int i = 0; i < DK; ++i) {
            float x = src ? src[(int64_t)i * DV + col] : 0.f;
            if (MB) x = (i == col) ? 1.f : 0.f;
            S[i] = x;
        }
    }
    auto nonzero = [&]() -> bool {
        uint32_t acc = 0u;
#pragma unroll
        for (int i = 0; i < DK; ++i) acc |= f32_bits(S[i]) & 0x7fffffffu;
        return __ballot(acc != 0u) != 0ull;
    };
    auto store = [&](float *dst, const float *add) {
#pragma unroll
        for (int i = 0; i < DK; ++i) {
            const int64_t e = (int64_t)i * ldst + col;
            dst[e] = S[i] + (add ? add[e] : 0.f);
        }
    };
    const int64_t pbase = (MODE == kModePrefill && a.pos0) ? a.pos0[u] : 0;
    // rung stores after the first p tokens of the unit (p a multiple of the chunk)
    auto rung = [&](int64_t p) {
        if (a.interval <= 0) return;
        if (MODE == kModePrefill && a.ckpt_S) {
            if ((pbase + p) % a.interval == 0) {
                const int64_t row = (a.ckpt_off ? a.ckpt_off[u] : 0) + (pbase + p) / a.interval -
                                    pbase / a.interval - 1;
                store(a.ckpt_S + (row * H + h) * DK * DV, nullptr);
            }
        }
        const int64_t ap = t0 + p;   // sequence-relative (one sequence)
        if ((MODE == kModePackage || MODE == kModePackageM) && ap % a.interval == 0) {
            float *dst = MB ? a.ckpt_M : a.ckpt_S;
            if (dst) store(dst + ((ap / a.interval - 1) * H + h) * (int64_t)DK * ldst, nullptr);
        }
        if (MODE == kModeFixup && a.ckpt_S && ap % a.interval == 0) {
            const int64_t off = ((ap / a.interval - 1) * H + h) * (int64_t)DK * DV;
            store(a.ckpt_S + off, a.ckpt_in + off);
        }
    };
    // rungs after position `from` once the state is exactly zero
    auto zero_rungs_after = [&](int64_t from) {
        if (a.interval <= 0) return;
        for (int64_t ap = (from / a.interval + 1) * a.interval; ap <= t1; ap += a.interval) {
            const int64_t row = ap / a.interval - 1;
            if (MB && a.ckpt_M) {
#pragma unroll
                for (int i = 0; i < DK; ++i) a.ckpt_M[(row * H + h) * DK * DK + (int64_t)i * DK + col] = 0.f;
            }
            if (MODE == kModeFixup && a.ckpt_S && a.ckpt_S != a.ckpt_in) {
                const int64_t off = (row * H + h) * (int64_t)DK * DV;
#pragma unroll
                for (int i = 0; i < DK; ++i) {
                    const int64_t e = off + (int64_t)i * DV + col;
                    a.ckpt_S[e] = a.ckpt_in[e];
                }
            }
        }
    };
    if (CHECK0 && !nonzero()) {   // nothing to propagate
        zero_rungs_after(t0);
        if (MB) store(package_slot(a.M_out, a.M_last, a.X_per, u, H, h, DK * DK), nullptr);
        return;
    }
    for (int64_t t = 0; t < len; ++t) {
        const int64_t tok = t0 + t;
        const int64_t base = (tok * H + h) * DK;
        // normalised k, q and alpha, two channels per lane, through LDS
        {
            const float k0 = ((const float *)a.k)[base + lane], k1 = ((const float *)a.k)[base + 64 + lane];
            float q0 = 0.f, q1 = 0.f;
            if (HAS_O) {
                q0 = ((const float *)a.q)[base + lane];
                q1 = ((const float *)a.q)[base + 64 + lane];
            }
            const float g0 = a.g[base + lane], g1 = a.g[base + 64 + lane];
            float sk = k0 * k0 + k1 * k1, sq = q0 * q0 + q1 * q1;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                sk += __shfl_xor(sk, off);
                sq += __shfl_xor(sq, off);
            }
            const float fk = a.l2norm ? 1.f / sqrtf(sk + 1e-6f) : 1.f;
            const float fq = a.l2norm ? a.scale / sqrtf(sq + 1e-6f) : a.scale;
            __syncthreads();   // the previous token's reads are done
            s_k[lane] = k0 * fk;
            s_k[lane + 64] = k1 * fk;
            s_q[lane] = q0 * fq;
            s_q[lane + 64] = q1 * fq;
            s_a[lane] = expf(g0);
            s_a[lane + 64] = expf(g1);
            __syncthreads();
        }
        const float beta = a.beta[tok * H + h];
        float vj = 0.f;
        if (HAS_V) vj = ((const float *)a.v)[(tok * H + h) * DV + col];
        float r = 0.f;
#pragma unroll
        for (int i = 0; i < DK; ++i) {
            S[i] *= s_a[i];
            r = fmaf(S[i], s_k[i], r);
        }
        const float uj = beta * (vj - r);
        float o = 0.f;
#pragma unroll
        for (int i = 0; i < DK; ++i) {
            S[i] = fmaf(s_k[i], uj, S[i]);
            o = fmaf(S[i], s_q[i], o);
        }
        if (HAS_O) {
            float *op = (float *)a.o + (tok * H + h) * DV + col;
            *op = (MODE == kModeFixup) ? *op + o : o;
        }
        const int64_t p = t + 1;
        if (p % kChunk == 0) {
            rung(p);
            if (CHECK0 && p < len && !nonzero()) {   // exact zero: stays zero
                zero_rungs_after(t0 + p);
                if (MB) store(package_slot(a.M_out, a.M_last, a.X_per, u, H, h, DK * DK), nullptr);
                return;
            }
        }
    }
    if (MODE == kModePrefill) {
        float *dst = nullptr;
        if (a.s_out_idx) {
            const int32_t slot = a.s_out_idx[u];
            if (slot >= 0 && slot < a.n_slots) dst = a.S_out + ((int64_t)slot * H + h) * DK * DV;
        } else if (a.S_out) {
            dst = a.S_out + ((int64_t)u * H + h) * DK * DV;
        }
        if (dst) store(dst, nullptr);
    }
    if (MODE == kModePackage || MODE == kModePackageM) {
        if (MB) store(package_slot(a.M_out, a.M_last, a.X_per, u, H, h, DK * DK), nullptr);
        else store(package_slot(a.S_out, a.S_last, a.X_per, u, H, h, DK * DV), nullptr);
    }
}

// One wave per (unit, head, column block); the package mode's M blocks
// follow its value blocks in the same grid (grid_v = value waves).
template <int DK, int DV, int MODE>
__global__ __launch_bounds__(64) void recurrent_kernel(EngineArgs a, int grid_v) {
    const int H = a.H;
    const bool mblk = MODE == kModePackageVM && (int)blockIdx.x >= grid_v;
    const int ncb = mblk ? a.ncb_m : a.ncb;
    const int bx = mblk ? (int)blockIdx.x - grid_v : (int)blockIdx.x;
    const int cb = bx % ncb;
    const int item = bx / ncb;
    if (item >= a.n_units * H) return;
    const int pos = item / H;
    const int h = item - pos * H;
    const int u = a.order ? a.order[pos] : pos;
    const int64_t t0 = a.bounds[u], t1 = a.bounds[u + 1];
    if (MODE == kModePackageVM) {
        if (mblk) recurrent_body<DK, DV, kModePackageM, true>(a, u, h, cb * kCols, t0, t1);
        else recurrent_body<DK, DV, kModePackage, false>(a, u, h, cb * kCols, t0, t1);
    } else {
        recurrent_body<DK, DV, MODE, MODE == kModePackageM>(a, u, h, cb * kCols, t0, t1);
    }
}

template <int DK, int DV, int MODE>
hipError_t launch_rec(const EngineArgs &a, hipStream_t s) {
    const int64_t items = (int64_t)a.n_units * a.H;
    const int64_t grid_v = items * a.ncb;
    const int64_t grid = grid_v + (MODE == kModePackageVM ? items * a.ncb_m : 0);
    if (grid == 0) return hipSuccess;
    if (grid > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL((recurrent_kernel<DK, DV, MODE>), dim3((unsigned)grid), dim3(64), 0, s, a,
                       (int)grid_v);
    return hipGetLastError();
}

}  // namespace

bool recurrent_supported(bool bf16, int dk, int dv) {
    return !bf16 && dk == 128 && (dv == 64 || dv == 128);
}

// a.ncb = dv / 64 value-column waves (a.ncb_m = dk / 64 for the M blocks).
hipError_t launch_recurrent(int mode, int dk, int dv, const EngineArgs &a, hipStream_t s) {
    if (dk != 128 || (dv != 64 && dv != 128) || a.ncb * kCols != dv) return hipErrorInvalidValue;
#define KDA_REC_MODES(DV_)                                                         \
    switch (mode) {                                                                \
        case kModePrefill: return launch_rec<128, DV_, kModePrefill>(a, s);        \
        case kModePackage: return launch_rec<128, DV_, kModePackage>(a, s);        \
        case kModeFixup: return launch_rec<128, DV_, kModeFixup>(a, s);            \
        case kModePackageM: return launch_rec<128, DV_, kModePackageM>(a, s);      \
        case kModePackageVM: return launch_rec<128, DV_, kModePackageVM>(a, s);    \
    }
    if (dv == 64) {
        KDA_REC_MODES(64)
    } else {
        KDA_REC_MODES(128)
    }
#undef KDA_REC_MODES
    return hipErrorInvalidValue;
}

}  // namespace kda
