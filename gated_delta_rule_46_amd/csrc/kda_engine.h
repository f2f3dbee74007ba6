// kda_engine.h -- warp-specialised chunkwise KDA engine for gfx950 (MI355X).
//
// Included by one translation unit per (dk, dv) shape family (kda_chunk_*.hip),
// which instantiate the engine for their shapes; kda_chunk.hip dispatches.
//
// One workgroup (8 wave64s) walks one (unit, head, column block) through its
// chunks of 64 tokens in order.  A unit is a sequence (prefill) or a segment
// (package / fix-up).  The waves split into two roles that run concurrently:
//
//   producers (waves 0-3, one per 16-row block b of the chunk) prepare chunk
//     c+1: loads of q, k, g, beta (prefetched one chunk ahead), L2 norms,
//     in-block cumulative log2-decay, exponentials, the Gram matrices A and P
//     and the diagonal inverses T_bb on the matrix cores;
//   consumers (waves 4-7) own a quarter of the state's columns each (fp32 MFMA
//     accumulators), read their value columns of V themselves, and apply
//     chunk c:
//         U = (I + A)^-1 (beta V - R_k S)       R_k = beta K*Gam
//         O = (Q*Gam) S + P U,   S <- Diag(gamma_C) S + Kbar^T U.
//
// Two workgroup barriers per chunk.  Between the second barrier and the first
// the consumers apply chunk c while the producers prepare all of chunk c+1:
// norms, decay scan and block totals; then, once the four producers have
// published their totals (a counter in LDS), the per-channel factors, the
// hand-off tiles already rescaled to the chunk start, the diagonal Gram
// blocks, T_bb = (I + A_bb)^-1 on the fp32 matrix core and, after a second
// counter, the off-diagonal blocks.  Every tile written in that phase (-R_k,
// Kbar^T, P, -A, T_bb) has two copies, by chunk parity.  Between the first
// barrier and the second the producers only copy the single-copy tiles (Qbar,
// beta, gamma; -R_k where LDS holds one copy only) from registers while the
// consumers store checkpoint rungs and run the zero test.
//
// Numerical scheme: one reference point per 16-row block.  The diagonal block
// uses the block start (lhs factor <= 1, rhs factor <= e^{span of 16 tokens}),
// off-diagonal blocks use the end of the earlier block (all factors <= 1).
// Valid while a channel's log-decay over any aligned 16 tokens stays above
// about -80.  Per element only two exponentials are evaluated; every other
// factor is a per-channel constant computed once per channel.
//
// The chunkwise algebra is derived from the KDA recurrence (pegainfer PR #970
// names the (M,D) segment packages built on it; the chunk form is the WY / UT
// form of the delta rule).

#pragma once

#include <atomic>
#include <type_traits>

#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {
namespace {

using namespace mf;

constexpr int kThreads = 512;

// Destination of the output stores of padded rows (rows past the end of a
// unit in its last chunk): the stores stay unconditional, so the compiler's
// wait counts for the value-row loads issued before them stay exact.  Nothing
// reads it; concurrent writes of discarded values are harmless.
__device__ __align__(16) uint32_t g_discard[64 * 4 * 2];

// Compact storage of the six strictly-lower 16x16 blocks (b, a), a < b.
__host__ __device__ constexpr int aoff_idx(int b, int a) { return b * (b - 1) / 2 + a; }

template <int DK, int NB, bool BF, int RKN_> struct LdsL {
    using T = typename Ops<BF>::T;
    // Row padding.  Tiles that the consumers read as 8-byte fragments (two
    // per operand) keep a row stride of 2 mod 4 dwords in bf16: gfx950 serves
    // an 8-byte LDS access 16 lanes at a time over 32 four-byte banks, so the
    // 16 rows of a fragment then fall on 16 distinct bank pairs (a stride of
    // 0 mod 4 dwords puts rows m and m+8 on the same pair).  Those rows are
    // only 8-byte aligned and are written with 8-byte stores.  Producer-only
    // tiles, read and written 16 bytes per lane, use a stride of 8 mod 16
    // dwords, which measured free of conflicts for 16-byte accesses.
    static constexpr int PAD = BF ? 4 : Ops<BF>::PAD;
    static constexpr int PADR = BF ? 16 : Ops<BF>::PAD;
    static constexpr int ES = (int)sizeof(T);
    static constexpr int LDQ = DK + PAD;        // [64][DK] row-major tiles
    static constexpr int LDK = 64 + PAD;        // [DK][64] transposed Kbar
    static constexpr int LDP = 64 + PAD;        // [64][64] P
    static constexpr int LDT = 16 + PAD;        // 16x16 blocks
    static constexpr int LDR = DK + PADR;       // producer-side [rows][DK] tiles
    static constexpr int o_flag = 0;                                  // int[16]: consumer zero flags
    static constexpr int o_sync = 64;                                 // int[8]: producer counters
    static constexpr int o_gam = 96;                                  // f32 [DK]
    static constexpr int o_tot = o_gam + DK * 4;                      // f32 [4][DK]
    static constexpr int o_fac = o_tot + 4 * DK * 4;                  // f32 [4][4][DK]
    static constexpr int o_qbar = o_fac + 16 * DK * 4;                // hand-off: Q Gam
    static constexpr int RKN = RKN_;
    static constexpr int o_rk = o_qbar + 64 * LDQ * ES;               // hand-off: -R_k [RKN]
    static constexpr int o_kbt = o_rk + RKN * 64 * LDQ * ES;          // hand-off: Kbar^T [2]
    static constexpr int o_beta = o_kbt + 2 * DK * LDK * ES;          // hand-off: beta [64] f32
    static constexpr int o_p = o_beta + 64 * 4;                       // hand-off: P [2]
    static constexpr int o_aoff = o_p + 2 * 64 * LDP * ES;            // hand-off: -A blocks [2]
    static constexpr int o_td = o_aoff + 2 * 6 * 16 * LDT * ES;       // hand-off: T_bb [2][4]
    static constexpr int o_ro = o_td + 2 * 4 * 16 * LDT * ES;         // rhs of blocks 0-2
    static constexpr int o_lk = o_ro + 48 * LDR * ES;                 // lhs (K) of block 2
    static constexpr int o_lq = o_lk + 16 * LDR * ES;                 // lhs (Q) of block 2
    static constexpr int size = o_lq + 16 * LDR * ES;
    static constexpr int P_BUF = 64 * LDP;                            // elements per buffer
    static constexpr int AOFF_BUF = 6 * 16 * LDT;
    static constexpr int TD_BUF = 4 * 16 * LDT;
    static constexpr int KBT_BUF = DK * LDK;
    static constexpr int RK_BUF = 64 * LDQ;
    static_assert(o_gam % 16 == 0 && o_qbar % 16 == 0 && o_rk % 16 == 0 && o_kbt % 16 == 0 &&
                  o_p % 16 == 0 && o_beta % 16 == 0 && o_aoff % 16 == 0 && o_td % 16 == 0 &&
                  o_ro % 16 == 0 && o_lk % 16 == 0 && o_lq % 16 == 0 && (P_BUF * ES) % 16 == 0 &&
                  (AOFF_BUF * ES) % 16 == 0 && (TD_BUF * ES) % 16 == 0, "LDS alignment");
    static_assert((LDQ * ES) % 8 == 0 && (LDK * ES) % 8 == 0 && (LDP * ES) % 8 == 0 &&
                  (LDT * ES) % 8 == 0 && (LDR * ES) % 16 == 0,
                  "row alignment of 8-byte and 16-byte LDS accesses");
};
// -R_k is double-buffered (written in the own phase) where the LDS budget
// allows it, else single (written from registers between the barriers).
template <int DK, int NB, bool BF>
using Lds = typename std::conditional<(LdsL<DK, NB, BF, 2>::size <= 160 * 1024), LdsL<DK, NB, BF, 2>,
                                      LdsL<DK, NB, BF, 1>>::type;

// Producer counters in LDS.  A producer publishes chunk c once its LDS writes
// of that chunk are done (LDS operations of a wave complete in order, so a
// wait on the LDS counter suffices; no wait on its outstanding global loads),
// and waits until the other producers have published chunk c.  All waves of a
// workgroup are resident together, so the waits end; the wait is bounded all
// the same (2^16 polls), so that a broken protocol shows as wrong values
// rather than as a hang.
typedef __attribute__((address_space(3))) int lds_int;
__device__ __forceinline__ void publish(int *cnt, int c) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if ((threadIdx.x & 63) == 0)
        __hip_atomic_store((lds_int *)cnt, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void wait_all4(const int *cnt, int c) {
    for (int it = 0; it < (1 << 16); ++it) {
        lds_int *p = (lds_int *)cnt;
        const int a = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        const int b = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        const int d = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(p + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        const int e = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(p + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (a >= c && b >= c && d >= c && e >= c) break;
        __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
}

// T = (I + N)^-1 for a strictly lower 16x16 N, from N and N^T in the MFMA
// accumulator layout (lane (n, g) element i: row 4g+i, column n), as
// (I - N)(I + N^2)(I + N^4)(I + N^8), exact for N^16 = 0, on the fp32 matrix
// core: X1 = I + N^4 + N^8 + N^4 N^8, X2 = X1 + N^2 X1, T = X2 - N X2.
// mul(X^T, Y) = X Y: with k = 4g + s, the B operand of step s is element s
// of Y's accumulator and the A operand element s of X^T's.
__device__ __forceinline__ f32x4 mul_acc(f32x4 xt, f32x4 y) {
    f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) r = __builtin_amdgcn_mfma_f32_16x16x4f32(xt[s], y[s], r, 0, 0, 0);
    return r;
}
__device__ __forceinline__ f32x4 inv_unit_lower(f32x4 N, f32x4 Nt, int n, int g) {
    f32x4 I;
#pragma unroll
    for (int i = 0; i < 4; ++i) I[i] = (4 * g + i == n) ? 1.f : 0.f;
    const f32x4 N2 = mul_acc(Nt, N), N2t = mul_acc(N, Nt);
    const f32x4 N4 = mul_acc(N2t, N2), N4t = mul_acc(N2, N2t);
    const f32x4 N8 = mul_acc(N4t, N4);
    const f32x4 X1 = I + N4 + N8 + mul_acc(N4t, N8);
    const f32x4 X2 = X1 + mul_acc(N2t, X1);
    return X2 - mul_acc(Nt, X2);
}

// Raw rows of one chunk held in registers between the prefetch and its use.
template <bool BF, int KS> struct Raw {
    static constexpr int W8 = BF ? 4 : 8;      // 32-bit words per 8 elements
    uint32_t q[KS * W8], k[KS * W8], g[KS * 8];
    float b;
};

template <bool BF>
__device__ __forceinline__ void ld_words(const void *base, int64_t idx, uint32_t *w) {
    if (BF) {
        const uint4 x = *(const uint4 *)((const __bf16 *)base + idx);
        w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    } else {
        const uint4 x = *(const uint4 *)((const float *)base + idx);
        const uint4 y = *(const uint4 *)((const float *)base + idx + 4);
        w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
        w[4] = y.x; w[5] = y.y; w[6] = y.z; w[7] = y.w;
    }
}

template <bool BF>
__device__ __forceinline__ void unpack_words(const uint32_t *w, float *out) {
    if (BF) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            out[2 * j] = __builtin_bit_cast(float, w[j] << 16);
            out[2 * j + 1] = __builtin_bit_cast(float, w[j] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) out[j] = bits_f32(w[j]);
    }
}

template <int DKT, int NTW>
__device__ __forceinline__ void store_state(float *dst, int ld, int col0, int gq, int m,
                                            const f32x4 (&S)[DKT][NTW], bool zero) {
#pragma unroll
    for (int r = 0; r < DKT; ++r)
#pragma unroll
        for (int n = 0; n < NTW; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dst[(int64_t)(16 * r + 4 * gq + i) * ld + col0 + 16 * n + m] = zero ? 0.f : S[r][n][i];
}

// dst = S + add at the state positions this lane owns (add laid out like
// dst).  Two row tiles at a time, every load of a batch before its stores:
// dst and add may alias as far as the compiler knows, so interleaved
// accesses would each wait a full memory round trip.
template <int DKT, int NTW>
__device__ __forceinline__ void store_state_add(float *dst, const float *add, int ld, int col0,
                                                int gq, int m, const f32x4 (&S)[DKT][NTW]) {
    static_assert(DKT % 2 == 0, "row tiles in pairs");
#pragma unroll
    for (int r0 = 0; r0 < DKT; r0 += 2) {
        float x[2][NTW][4];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    x[r][n][i] = add[(int64_t)(16 * (r0 + r) + 4 * gq + i) * ld + col0 + 16 * n + m];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dst[(int64_t)(16 * (r0 + r) + 4 * gq + i) * ld + col0 + 16 * n + m] =
                        S[r0 + r][n][i] + x[r][n][i];
    }
}

// dst = src over rows [0, DK) and columns [col0, col0 + NB) of a [DK x ld]
// state, by the 256 threads of the consumer waves (ct = 0..255), 16 bytes per
// access, every load before any store.
template <int DK, int NB>
__device__ __forceinline__ void copy_state_block(float *dst, const float *src, int ld, int col0,
                                                 int ct) {
    constexpr int Q = NB / 4;                  // float4 per row
    constexpr int PER = DK * Q / 256;
    static_assert(PER * 256 == DK * Q, "block shape");
    f32x4 t[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int idx = ct + 256 * i, row = idx / Q, c4 = idx - row * Q;
        t[i] = *(const f32x4 *)(src + (int64_t)row * ld + col0 + 4 * c4);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int idx = ct + 256 * i, row = idx / Q, c4 = idx - row * Q;
        *(f32x4 *)(dst + (int64_t)row * ld + col0 + 4 * c4) = t[i];
    }
}

// Some consumer wave flagged a nonzero state (four consumer waves).
__device__ __forceinline__ bool s_flag_any(const unsigned char *smem) {
    const int *f = (const int *)smem;
    return (f[0] | f[1] | f[2] | f[3]) != 0;
}

template <int MODE, bool MB> struct Roles {
    static constexpr bool HAS_V = (MODE != kModeFixup) && !MB;   // beta V enters U
    static constexpr bool HAS_O = !MB;                           // outputs are produced
    static constexpr bool CHECK0 = (MODE == kModeFixup) || MB;   // stop once S is exactly 0
};

// The operator that the M block of unit u writes.  Unsplit units and the
// first sub-segment of a split segment write their segment's (X, at u /
// X_per); a later sub-segment writes its own (Xs, when given).  `whole`: the
// operator covers the block's unit and no more, so a count at the block's end
// is valid without the identity having vanished.
struct XOut {
    void *X;
    int32_t *len;
    float *Pi;
    int64_t slot;
    int chunks, interval;
    bool whole;
};
__device__ __forceinline__ XOut x_out(const EngineArgs &a, int u) {
    if (a.X_per > 1 && u % a.X_per != 0)
        return {a.Xs, a.Xs_len, a.Xs_Pi,
                (int64_t)(u % a.X_per - 1) * (a.n_units / a.X_per) + u / a.X_per, a.Xs_chunks,
                a.Xs_interval, true};
    return {a.X, a.X_len, a.X_Pi, a.X_per > 1 ? u / a.X_per : u, a.X_chunks, a.X_interval,
            a.X_per <= 1};
}

// Fix-up of a unit [t0, t1) from the operator X at index xu (fixop_kernel):
// the chunks of rows to correct, or -1 when the unit walks the recurrence
// instead.  That is the case
// with no operator; with a 64-column block whose identity had not vanished
// within X_chunks chunks, or a count outside [0, X_chunks] (the bound keeps
// every row of X read in range); with an incoming state holding an infinity or
// a NaN (bit 1 of flags); and with a checkpoint rung among the corrected rows
// that the operator's Pi does not cover.  Pi covers only the first rung after
// the segment start, and only at the operator's interval; a second rung among
// the rows needs the recurrence.  pi_rung returns the covered rung (or -1).
template <int DK>
__device__ __forceinline__ int fixup_x_chunks(const EngineArgs &a, int xu, int h, int64_t t0,
                                              int64_t t1, int flags, int64_t &pi_rung) {
    pi_rung = -1;
    if (!a.X || !a.X_len || (flags & 2)) return -1;
    int lmax = 0;
#pragma unroll
    for (int j = 0; j < DK / 64; ++j) {
        const int l = a.X_len[((int64_t)xu * a.H + h) * (DK / 64) + j];
        if (l < 0 || l > a.X_chunks) return -1;
        lmax = l > lmax ? l : lmax;
    }
    if (a.ckpt_S && a.interval > 0 && lmax > 0) {
        const int64_t first = (t0 / a.interval + 1) * a.interval;
        const int64_t end = t0 + (int64_t)lmax * kChunk;   // the propagated identity is 0 here
        if (first <= t1 && first < end) {
            if (!a.X_Pi || a.X_interval != a.interval || first + a.interval < end) return -1;
            pi_rung = first;
        }
    }
    return lmax;
}

// ===========================================================================
// Producer wave for row block B of every chunk.
// ===========================================================================
template <int DK, int DV, int NB, bool BF, int MODE, bool MB, int B>
__device__ __forceinline__ void producer(const EngineArgs &a, unsigned char *smem, const int u,
                                         const int h,
                                         const int cbase, const int64_t t0, const int64_t t1,
                                         const int nchunks) {
    using O = Ops<BF>;
    using T = typename O::T;
    using F8 = typename O::F8;
    using F4 = typename O::F4;
    using L = Lds<DK, NB, BF>;
    using R = Roles<MODE, MB>;
    constexpr int KS = DK / 32;      // 32-channel steps of a row
    // M blocks with a fix-up operator also form the outputs of its first
    // chunks (the rows of X); other M blocks form none.
    const int xch = MB ? (x_out(a, u).X ? x_out(a, u).chunks : 0) : 0;
    auto out_on = [&](int c) { return R::HAS_O || c < xch; };
    constexpr int W8 = BF ? 4 : 8;

    int *s_sync = (int *)(smem + L::o_sync);
    float *s_gam = (float *)(smem + L::o_gam);
    float *s_tot = (float *)(smem + L::o_tot);
    float *s_fac = (float *)(smem + L::o_fac);
    T *s_qbar = (T *)(smem + L::o_qbar);
    T *s_rk = (T *)(smem + L::o_rk);
    T *s_kbt = (T *)(smem + L::o_kbt);
    T *s_p = (T *)(smem + L::o_p);
    float *s_beta = (float *)(smem + L::o_beta);
    T *s_aoff = (T *)(smem + L::o_aoff);
    T *s_td = (T *)(smem + L::o_td);
    T *s_ro = (T *)(smem + L::o_ro);
    T *s_lk = (T *)(smem + L::o_lk);
    T *s_lq = (T *)(smem + L::o_lq);

    const int lane = threadIdx.x & 63;
    const int H = a.H;

    // Blocks of P right of the diagonal are zero in every chunk (both buffers).
    if (R::HAS_O || xch > 0) {
        const int m = lane & 15, gq = lane >> 4;
#pragma unroll
        for (int pb = 0; pb < 2; ++pb)
#pragma unroll
            for (int a2 = B + 1; a2 < 4; ++a2)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s_p[pb * L::P_BUF + (16 * B + 4 * gq + i) * L::LDP + 16 * a2 + m] = (T)0.f;
    }
    // Identity selectors: an MFMA of a row-layout fragment with isel[hh]
    // returns channels 16hh..16hh+15 of the 32-channel step transposed.
    F8 isel[2];
    {
        const int n = lane & 15, g = lane >> 4;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            float e[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) e[j] = (8 * g + j == 16 * hh + n) ? 1.f : 0.f;
            isel[hh] = O::cvt8(e);
        }
    }

    Raw<BF, KS> raw;
    bool raw_valid = false;
    int64_t ld_tok = t0;
    // Rows of chunk c.  A row past the end of the unit is read from the unit's
    // first row (always in bounds) and masked to zero when used, so the loads
    // need no branches.
    auto set_rows = [&](int c) {
        const int m = opaque(lane) & 15;
        const int64_t r = t0 + (int64_t)c * kChunk + 16 * B + m;
        raw_valid = r < t1;
        ld_tok = raw_valid ? r : t0;
    };
    auto issue_g = [&]() {
        const int gq = opaque(lane) >> 4;
        const int64_t base = (ld_tok * H + h) * DK;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) ld_words<false>(a.g, base + 32 * kk + 8 * gq, &raw.g[8 * kk]);
        raw.b = a.beta[ld_tok * H + h];
    };
    auto issue_kq = [&](int c) {   // rows of chunk c (set_rows(c) before)
        const int gq = opaque(lane) >> 4;
        const int64_t base = (ld_tok * H + h) * DK;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) ld_words<BF>(a.k, base + 32 * kk + 8 * gq, &raw.k[W8 * kk]);
        if (out_on(c)) {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) ld_words<BF>(a.q, base + 32 * kk + 8 * gq, &raw.q[W8 * kk]);
        }
    };
    // Fragments of chunk c kept in registers from the own phase to the
    // hand-off phase: lhs of the Gram blocks (block-start reference), the
    // single-buffered hand-off tiles already rescaled to the chunk start, and
    // e^{G_C} of this lane's channels (block 0).
    F8 lhsK[KS], lhsQ[KS], qbf[KS], rkf[L::RKN == 1 ? KS : 1];
    float gamr[DK / 64], btc = 0.f;

    // An off-diagonal block (B2, A2) of A and P: lhs rows of block B2 (lk,
    // lq, referenced to the end of block B2-1) times rhs rows of block A2
    // (s_ro, referenced to the end of block A2), times e^{rho_{B2-1} -
    // rho_{A2}} per channel when the blocks are not adjacent (cf != null);
    // with po also the block of P.
    auto offdiag = [&](int buf, int B2, int A2, const F8 *lk, const F8 *lq, const T *lkp,
                       const T *lqp, const float *cf, bool po) {
        const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
        f32x4 Ao = {0.f, 0.f, 0.f, 0.f}, P_ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const int c0 = 32 * kk + 8 * gq;
            F8 Bf = O::ld8(s_ro + (16 * A2 + m) * L::LDR + c0);
            if (cf) {
                float x[8];
                O::unpack8(Bf, x);
                const f32x4 f0 = *(const f32x4 *)(cf + c0), f1 = *(const f32x4 *)(cf + c0 + 4);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) { x[jj] *= f0[jj]; x[jj + 4] *= f1[jj]; }
                Bf = O::cvt8(x);
            }
            const F8 Kf = lk ? lk[kk] : O::ld8(lkp + m * L::LDR + c0);
            Ao = O::mma32(Ao, Kf, Bf);
            if (po) {
                const F8 Qf = lq ? lq[kk] : O::ld8(lqp + m * L::LDR + c0);
                P_ = O::mma32(P_, Qf, Bf);
            }
        }
        T *dst = s_aoff + buf * L::AOFF_BUF + aoff_idx(B2, A2) * 16 * L::LDT;
        T *pd = s_p + buf * L::P_BUF;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dst[(4 * gq + i) * L::LDT + m] = (T)(-Ao[i]);
            if (po) pd[(16 * B2 + 4 * gq + i) * L::LDP + 16 * A2 + m] = (T)P_[i];
        }
    };

    // All the work of chunk c (runs while the consumers apply chunk c-1).
    auto phase_own = [&](int c) {
        const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
        const int prow = 16 * B + m;
        const int buf = c & 1;
        const bool more = c + 1 < nchunks;
        const bool partial = t0 + (int64_t)(c + 1) * kChunk > t1;
        const bool oc = out_on(c);   // the outputs' tiles (Qbar, P) of chunk c
        const float vm = raw_valid ? 1.f : 0.f;
        float gl[KS * 8];
#pragma unroll
        for (int e = 0; e < KS * 8; ++e) gl[e] = bits_f32(raw.g[e]);
        if (partial) {   // padded rows act as identity: g = 0, k = q = v = 0, beta = 0
#pragma unroll
            for (int e = 0; e < KS * 8; ++e) gl[e] *= vm;
        }
        const float bt = raw.b * vm;
#pragma unroll
        for (int e = 0; e < KS * 8; ++e) gl[e] = scan16(gl[e] * kLog2e);
        if (m == 15) {   // block totals, published for the other producers
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                float *d = s_tot + B * DK + 32 * kk + 8 * gq;
                *(f32x4 *)d = f32x4{gl[8 * kk], gl[8 * kk + 1], gl[8 * kk + 2], gl[8 * kk + 3]};
                *(f32x4 *)(d + 4) = f32x4{gl[8 * kk + 4], gl[8 * kk + 5], gl[8 * kk + 6], gl[8 * kk + 7]};
            }
        }
        publish(s_sync + B, c);
        float fk, fq = 0.f;
        if constexpr (BF) {
            // |row|^2 of the raw bf16 rows as the diagonal of their 16x16 Gram
            // block on the matrix core; entry (r, r) sits in lane r + 16*(r/4),
            // element r % 4.
            f32x4 Gk = {0.f, 0.f, 0.f, 0.f}, Gq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const bf16x8 kf = __builtin_bit_cast(bf16x8, *(const uint4 *)&raw.k[W8 * kk]);
                Gk = O::mma32(Gk, kf, kf);
                if (oc) {
                    const bf16x8 qf = __builtin_bit_cast(bf16x8, *(const uint4 *)&raw.q[W8 * kk]);
                    Gq = O::mma32(Gq, qf, qf);
                }
            }
            const int src = m + 16 * (m >> 2), e = m & 3;
            const float dk = e == 0 ? Gk[0] : e == 1 ? Gk[1] : e == 2 ? Gk[2] : Gk[3];
            fk = (a.l2norm ? rsqrtf(__shfl(dk, src) + kEps) : 1.f) * vm;
            if (oc) {
                const float dq = e == 0 ? Gq[0] : e == 1 ? Gq[1] : e == 2 ? Gq[2] : Gq[3];
                fq = (a.l2norm ? a.scale * rsqrtf(__shfl(dq, src) + kEps) : a.scale) * vm;
            }
        } else {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                float x[8];
                unpack_words<BF>(&raw.k[W8 * kk], x);
#pragma unroll
                for (int j = 0; j < 8; ++j) sk += x[j] * x[j];
                if (oc) {
                    unpack_words<BF>(&raw.q[W8 * kk], x);
#pragma unroll
                    for (int j = 0; j < 8; ++j) sq += x[j] * x[j];
                }
            }
            sk += __shfl_xor(sk, 16); sk += __shfl_xor(sk, 32);
            fk = (a.l2norm ? rsqrtf(sk + kEps) : 1.f) * vm;
            if (oc) {
                sq += __shfl_xor(sq, 16); sq += __shfl_xor(sq, 32);
                fq = (a.l2norm ? a.scale * rsqrtf(sq + kEps) : a.scale) * vm;
            }
        }
        btc = bt;
        if (more) {
            set_rows(c + 1);
            issue_g();
        }
        // Per-channel factors of block B (log2 domain, all <= 1); rho_a is the
        // decay at the end of block a, G_C the chunk's:
        //   [0] e^{tot_B} (rhs rows of later blocks; block 3: e^{tot_1+tot_2})
        //   [1] e^{rho_{B-1}} (Qbar, R_k)   [2] e^{G_C - rho_{B-1}} (Kbar)
        //   [3] block 0: e^{tot_1} (block (2,0)); block 3: e^{tot_2} (block (3,1))
        wait_all4(s_sync, c);
        float *fac = s_fac + B * 4 * DK;
#pragma unroll
        for (int i = 0; i < DK / 64; ++i) {
            const int ch = opaque(lane) + 64 * i;
            const float u0 = s_tot[ch], u1 = s_tot[DK + ch], u2 = s_tot[2 * DK + ch], u3 = s_tot[3 * DK + ch];
            const float rho = (B >= 1 ? u0 : 0.f) + (B >= 2 ? u1 : 0.f) + (B >= 3 ? u2 : 0.f);
            const float gc = u0 + u1 + u2 + u3;
            fac[ch] = ex2(B == 0 ? u0 : B == 1 ? u1 : B == 2 ? u2 : u1 + u2);
            if (B > 0) fac[DK + ch] = ex2(rho);
            fac[2 * DK + ch] = ex2(gc - rho);
            if (B == 0) fac[3 * DK + ch] = ex2(u1);
            if (B == 3) fac[3 * DK + ch] = ex2(u2);
            if (B == 0) gamr[i] = ex2(gc);
        }
        wave_sync_lds();
        const float fkb = fk * bt;
        f32x4 Ad = {0.f, 0.f, 0.f, 0.f}, Adt = {0.f, 0.f, 0.f, 0.f}, Pd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const int c0 = 32 * kk + 8 * gq;
            float e1[8], e2[8], kx[8], lk[8], rd[8], t8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) { e1[j] = ex2(gl[8 * kk + j]); e2[j] = ex2(-gl[8 * kk + j]); }
            unpack_words<BF>(&raw.k[W8 * kk], kx);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                lk[j] = kx[j] * fkb * e1[j];
                rd[j] = kx[j] * fk * e2[j];
            }
            lhsK[kk] = O::cvt8(lk);
            const F8 rhsD = O::cvt8(rd);
            if (B < 3) {   // rhs rows of later blocks, referenced to the end of block B
                const f32x4 f0 = *(const f32x4 *)(fac + c0), f1 = *(const f32x4 *)(fac + c0 + 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) { t8[j] = rd[j] * f0[j]; t8[j + 4] = rd[j + 4] * f1[j]; }
                O::st8(s_ro + prow * L::LDR + c0, t8);
            }
            {   // Kbar = rd * e^{G_C - rho_{B-1}}, transposed through the matrix core
                const f32x4 f0 = *(const f32x4 *)(fac + 2 * DK + c0), f1 = *(const f32x4 *)(fac + 2 * DK + c0 + 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) { t8[j] = rd[j] * f0[j]; t8[j + 4] = rd[j + 4] * f1[j]; }
                const F8 kbf = O::cvt8(t8);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    O::st4(s_kbt + buf * L::KBT_BUF + (32 * kk + 16 * hh + m) * L::LDK + 16 * B + 4 * gq,
                           O::mma32(f32x4{0.f, 0.f, 0.f, 0.f}, kbf, isel[hh]));
            }
            float f0r[8];   // e^{rho_{B-1}}
            if (B > 0) {
                const f32x4 f0 = *(const f32x4 *)(fac + DK + c0), f1 = *(const f32x4 *)(fac + DK + c0 + 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) { f0r[j] = f0[j]; f0r[j + 4] = f1[j]; }
            }
            {   // -R_k: -lk rescaled to the chunk start
                F8 r;
                if (B == 0) {
                    r = O::neg(lhsK[kk]);
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) t8[j] = -(lk[j] * f0r[j]);
                    r = O::cvt8(t8);
                }
                if constexpr (L::RKN == 2) O::stf_h(s_rk + buf * L::RK_BUF + prow * L::LDQ + c0, r);
                else rkf[kk] = r;
            }
            if (oc) {
                float qx[8], lq[8];
                unpack_words<BF>(&raw.q[W8 * kk], qx);
#pragma unroll
                for (int j = 0; j < 8; ++j) lq[j] = qx[j] * fq * e1[j];
                lhsQ[kk] = O::cvt8(lq);
                if (B == 0) {
                    qbf[kk] = lhsQ[kk];
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) t8[j] = lq[j] * f0r[j];
                    qbf[kk] = O::cvt8(t8);
                }
                Pd = O::mma32(Pd, lhsQ[kk], rhsD);
                if (B == 2) O::stf(s_lq + m * L::LDR + c0, lhsQ[kk]);
            }
            if (B == 2) O::stf(s_lk + m * L::LDR + c0, lhsK[kk]);
            Ad = O::mma32(Ad, lhsK[kk], rhsD);
            Adt = O::mma32(Adt, rhsD, lhsK[kk]);
            // one 32-channel step at a time keeps the fp32 temporaries short-lived
            __builtin_amdgcn_sched_barrier(0);
        }
        if (more) issue_kq(c + 1);
        publish(s_sync + 4 + B, c);   // s_ro (and block 2's lhs rows) written

        // T_bb = (I + A_bb)^-1 from the strictly lower part of A_bb
        {
            f32x4 N, Nt;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                N[i] = (m < 4 * gq + i) ? Ad[i] : 0.f;
                Nt[i] = (4 * gq + i < m) ? Adt[i] : 0.f;
            }
            const f32x4 Tb = inv_unit_lower(N, Nt, m, gq);
            T *td = s_td + buf * L::TD_BUF + B * 16 * L::LDT;
#pragma unroll
            for (int i = 0; i < 4; ++i) td[(4 * gq + i) * L::LDT + m] = (T)Tb[i];
        }
        if (oc) {   // diagonal block of P (lower triangle incl. the diagonal)
            T *pd = s_p + buf * L::P_BUF;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                pd[(16 * B + 4 * gq + i) * L::LDP + 16 * B + m] = (T)((m <= 4 * gq + i) ? Pd[i] : 0.f);
        }
        wait_all4(s_sync + 4, c);
        // Off-diagonal blocks: (B, B-1) needs no rescale (the rhs rows of
        // block B-1 are referenced to its end, where block B's lhs starts);
        // block 0 also forms (2,0) from block 2's lhs rows, block 3 also
        // (3,0) and (3,1).
        if (B >= 1) offdiag(buf, B, B - 1, lhsK, lhsQ, nullptr, nullptr, nullptr, oc);
        if (B == 0) offdiag(buf, 2, 0, nullptr, nullptr, s_lk, s_lq, fac + 3 * DK, oc);
        if (B == 3) {
            offdiag(buf, 3, 0, lhsK, lhsQ, nullptr, nullptr, fac, oc);
            offdiag(buf, 3, 1, lhsK, lhsQ, nullptr, nullptr, fac + 3 * DK, oc);
        }
    };

    // Hand-off of chunk c (between the barriers, while the consumers store
    // rungs): the single-buffered tiles, from registers.
    auto phase_cross = [&](int c) {
        const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
        const int prow = 16 * B + m;
        if (B == 0) {
#pragma unroll
            for (int i = 0; i < DK / 64; ++i) s_gam[opaque(lane) + 64 * i] = gamr[i];
        }
        if (out_on(c)) {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) O::stf_h(s_qbar + prow * L::LDQ + 32 * kk + 8 * gq, qbf[kk]);
        }
        if constexpr (L::RKN == 1) {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) O::stf_h(s_rk + prow * L::LDQ + 32 * kk + 8 * gq, rkf[kk]);
        }
        if (R::HAS_V && gq == 0) s_beta[prow] = btc;   // zero on padded rows
    };

    // prologue: chunk 0
    if (nchunks > 0) {
        set_rows(0);
        issue_g();
        issue_kq(0);
        phase_own(0);
    }
    __syncthreads();                                                          // BA
    if (nchunks > 0) phase_cross(0);
    __syncthreads();                                                          // BB
    for (int c = 0; c < nchunks; ++c) {
        if (R::CHECK0 && c > 0 && !(s_flag_any(smem))) return;
        const bool next = c + 1 < nchunks;
        if (next) phase_own(c + 1);
        __syncthreads();                                                      // BA
        if (next) phase_cross(c + 1);
        __syncthreads();                                                      // BB
    }
}

// ===========================================================================
// Consumer wave pw: state columns cbase + pw*NB/4 .. + NB/4 - 1.
// ===========================================================================
template <int DK, int DV, int NB, bool BF, int MODE, bool MB>
__device__ __forceinline__ void consumer(const EngineArgs &a, unsigned char *smem, const int u,
                                         const int h, const int cbase, const int64_t t0,
                                         const int64_t t1, const int nchunks, const int pw) {
    using O = Ops<BF>;
    using T = typename O::T;
    using F8 = typename O::F8;
    using F4 = typename O::F4;
    using L = Lds<DK, NB, BF>;
    using R = Roles<MODE, MB>;
    constexpr int KS = DK / 32;
    constexpr int NBW = NB / 4;      // state columns per consumer wave
    constexpr int NTW = NBW / 16;    // state column tiles per consumer wave
    constexpr int DKT = DK / 16;     // state row tiles
    constexpr int LDST = MB ? DK : DV;
    static_assert(NTW >= 1, "tile shape");
    // M blocks with a fix-up operator also form the outputs of its first
    // chunks, into its rows (the producers prepare their Qbar and P).
    const XOut xo = MB ? x_out(a, u) : XOut{};
    const int xch = MB && xo.X ? xo.chunks : 0;
    const int64_t ux = xo.slot;
    auto out_on = [&](int c) { return R::HAS_O || c < xch; };

    int *s_flag = (int *)(smem + L::o_flag);
    const float *s_gam = (const float *)(smem + L::o_gam);
    const T *s_qbar = (const T *)(smem + L::o_qbar);
    const T *s_rk = (const T *)(smem + L::o_rk);
    const T *s_kbt = (const T *)(smem + L::o_kbt);
    const T *s_p = (const T *)(smem + L::o_p);
    const float *s_beta = (const float *)(smem + L::o_beta);
    const T *s_aoff = (const T *)(smem + L::o_aoff);
    const T *s_td = (const T *)(smem + L::o_td);

    const int lane = threadIdx.x & 63;
    const int m = lane & 15, gq = lane >> 4;
    const int H = a.H;
    const int64_t len = t1 - t0;
    const int wcol = cbase + pw * NBW;

    f32x4 S[DKT][NTW];
    // rungs sit at absolute positions pbase + p (p sequence-relative)
    const int64_t pbase = (MODE == kModePrefill && a.pos0) ? a.pos0[u] : 0;
    {
        const float *src = nullptr;
        if (MODE == kModePrefill && a.s_in_idx) {
            const int32_t slot = a.s_in_idx[u];
            if (slot >= 0 && slot < a.n_slots) src = a.S_init + ((int64_t)slot * H + h) * DK * DV;
        } else if (MODE == kModePrefill && a.S_init) {
            src = a.S_init + (int64_t)(u * H + h) * DK * DV;
        }
        if (MODE == kModeFixup) src = a.S_init + (int64_t)(u * H + h) * DK * DV;
#pragma unroll
        for (int r = 0; r < DKT; ++r)
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * r + 4 * gq + i, col = wcol + 16 * n + m;
                    float val = src ? src[(int64_t)row * DV + col] : 0.f;
                    if (MB) val = (row == col) ? 1.f : 0.f;
                    S[r][n][i] = val;
                }
    }
    auto state_nonzero = [&]() -> bool {
        bool nz = false;
#pragma unroll
        for (int r = 0; r < DKT; ++r)
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    nz |= (f32_bits(S[r][n][i]) & 0x7fffffffu) != 0u;
        return __ballot(nz) != 0ull;
    };
    // Fix-up with rungs: once the propagated state is exactly zero, every
    // later rung p of the segment is its own part sub_D[p]; copied here for
    // the rungs after position `from`.
    auto copy_rungs_after = [&](int64_t from) {
        if (MODE != kModeFixup || !a.ckpt_S || a.interval <= 0 || a.ckpt_S == a.ckpt_in) return;
        for (int64_t p = (from / a.interval + 1) * a.interval; p <= t1; p += a.interval) {
            const int64_t off = ((p / a.interval - 1) * H + h) * DK * DV;
            copy_state_block<DK, NB>(a.ckpt_S + off, a.ckpt_in + off, DV, cbase,
                                     (int)threadIdx.x - 256);
        }
    };
    // Output rows of chunk c from the O^T tiles (four consecutive columns of
    // one token per lane, row-contiguous stores): to o, added to it in the
    // fix-up; for M blocks to the rows of X.  Padded rows store to the
    // discard array (no branch).
    auto put_rows = [&](int c, const f32x4 (&Ot)[4][NTW]) {
        const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
        const int64_t r0 = t0 + (int64_t)c * kChunk;
        unsigned char *base = MB ? (unsigned char *)xo.X : (unsigned char *)a.o;
#pragma unroll
        for (int mu = 0; mu < 4; ++mu) {
            const int64_t tok = r0 + 16 * mu + m;
            const bool valid = tok < t1;
            const int64_t row = MB ? (ux * xch * kChunk + (tok - t0)) * H + h
                                   : tok * H + h;
#pragma unroll
            for (int n = 0; n < NTW; ++n) {
                const int64_t idx = row * LDST + wcol + 16 * n + 4 * gq;
                f32x4 val = Ot[mu][n];
                uint32_t *dst = valid ? (uint32_t *)(base + idx * (BF ? 2 : 4)) : g_discard + 8 * lane;
                if (BF) {
                    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                    u32x2 *o = (u32x2 *)dst;
                    if (MODE == kModeFixup) {
                        const u32x2 w = *o;
                        val[0] += __builtin_bit_cast(float, w[0] << 16);
                        val[1] += __builtin_bit_cast(float, w[0] & 0xffff0000u);
                        val[2] += __builtin_bit_cast(float, w[1] << 16);
                        val[3] += __builtin_bit_cast(float, w[1] & 0xffff0000u);
                    }
                    *(bf16x4 *)o = Ops<true>::cvt4(val);
                } else {
                    f32x4 *o = (f32x4 *)dst;
                    if (MODE == kModeFixup) val += *o;
                    *o = val;
                }
            }
        }
    };
    if (MODE == kModeFixup) {
        // An all-zero incoming state leaves o_local final: skip the unit.
        const bool nz = state_nonzero();
        if (lane == 0) s_flag[pw] = nz ? 1 : 0;
        __syncthreads();
        const bool any = s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3];
        __syncthreads();
        if (!any) {
            copy_rungs_after(t0);
            return;
        }
    }

    // V enters U through a 16x16x16 MFMA with an identity selector, which
    // puts the rows of this wave's column tiles in the accumulator layout
    // (lane (m, gq) loads 4 consecutive columns of row m); beta scales the
    // result in fp32.  The rows of chunk c+1 are loaded while chunk c is
    // applied; rows past the end of the unit are read from its first row and
    // meet beta = 0.
    typename O::F4 isel16, vf[4][NTW];
    {
        float e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) e[j] = (4 * gq + j == m) ? 1.f : 0.f;
        isel16 = O::cvt4(f32x4{e[0], e[1], e[2], e[3]});
    }
    auto load_v = [&](int c) {
        if (!R::HAS_V) return;
        const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
#pragma unroll
        for (int mu = 0; mu < 4; ++mu) {
            const int64_t r = t0 + (int64_t)c * kChunk + 16 * mu + m;
            const int64_t tok = r < t1 ? r : t0;
#pragma unroll
            for (int n = 0; n < NTW; ++n)
                vf[mu][n] = *(const typename O::F4 *)((const T *)a.v + (tok * H + h) * DV + wcol +
                                                      16 * n + 4 * gq);
        }
    };
    if (nchunks > 0) load_v(0);

    // Applies chunk c: U, outputs, state update.
    auto apply = [&](int c) {
        const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
        F8 Sb[KS][NTW];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int n = 0; n < NTW; ++n) Sb[kk][n] = O::cvt44(S[2 * kk][n], S[2 * kk + 1][n]);
        // U = beta V - R_k S
        f32x4 U[4][NTW];
#pragma unroll
        for (int mu = 0; mu < 4; ++mu)
#pragma unroll
            for (int n = 0; n < NTW; ++n) U[mu][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mu = 0; mu < 4; ++mu) {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const T *p = s_rk + (L::RKN == 2 ? (c & 1) * L::RK_BUF : 0) + (16 * mu + m) * L::LDQ +
                             32 * kk + 4 * gq;
                const F8 Af = O::ld44(p, p + 16);
#pragma unroll
                for (int n = 0; n < NTW; ++n) U[mu][n] = O::mma32(U[mu][n], Af, Sb[kk][n]);
            }
            if (R::HAS_V) {   // U += beta * V (a separate chain: MFMA shapes never mix)
                const f32x4 b4 = *(const f32x4 *)(s_beta + 16 * mu + 4 * gq);
#pragma unroll
                for (int n = 0; n < NTW; ++n) {
                    const f32x4 vv = O::mma16(f32x4{0.f, 0.f, 0.f, 0.f}, vf[mu][n], isel16);
                    U[mu][n] = vv * b4 + U[mu][n];
                }
            }
        }
        if (c + 1 < nchunks) load_v(c + 1);
        // (I + A) X = U by block forward substitution; X overwrites U.  The
        // off-diagonal terms accumulate onto U with the same 32-deep MFMA that
        // produced U, two 16-blocks per instruction (a zero half where a block
        // row has an odd count): an accumulator chain must not switch MFMA
        // opcodes, gfx950 does not order a srcC read after a different-shape
        // MFMA that has just written it.  T_bb starts from a zero accumulator.
        const T *td = s_td + (c & 1) * L::TD_BUF;
        const T *aoff = s_aoff + (c & 1) * L::AOFF_BUF;
        const F4 z4 = O::cvt4(f32x4{0.f, 0.f, 0.f, 0.f});
        auto negA = [&](int b, int a2) { return O::ld4(aoff + (aoff_idx(b, a2) * 16 + m) * L::LDT + 4 * gq); };
        F4 Xb[4][NTW];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            F8 A01, A2;
            if (b == 1) A01 = O::cat(negA(1, 0), z4);
            if (b >= 2) A01 = O::cat(negA(b, 0), negA(b, 1));
            if (b == 3) A2 = O::cat(negA(3, 2), z4);
            const typename O::F4 Tf = O::ld4(td + (16 * b + m) * L::LDT + 4 * gq);
#pragma unroll
            for (int n = 0; n < NTW; ++n) {
                f32x4 Y = U[b][n];
                if (b == 1) Y = O::mma32(Y, A01, O::cat(Xb[0][n], z4));
                if (b >= 2) Y = O::mma32(Y, A01, O::cat(Xb[0][n], Xb[1][n]));
                if (b == 3) Y = O::mma32(Y, A2, O::cat(Xb[2][n], z4));
                U[b][n] = O::mma16(f32x4{0.f, 0.f, 0.f, 0.f}, Tf, O::cvt4(Y));
                Xb[b][n] = O::cvt4(U[b][n]);
            }
        }
        F8 Ub[2][NTW];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int n = 0; n < NTW; ++n) Ub[k2][n] = O::cat(Xb[2 * k2][n], Xb[2 * k2 + 1][n]);

        if (out_on(c)) {
            // O^T = S^T Qbar^T + U^T P^T: the MFMA output then holds four
            // consecutive columns of one token per lane (row-contiguous stores).
            f32x4 Ot[4][NTW];
#pragma unroll
            for (int mu = 0; mu < 4; ++mu)
#pragma unroll
                for (int n = 0; n < NTW; ++n) Ot[mu][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mu = 0; mu < 4; ++mu) {
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    const T *p = s_qbar + (16 * mu + m) * L::LDQ + 32 * kk + 4 * gq;
                    const F8 Bq = O::ld44(p, p + 16);
#pragma unroll
                    for (int n = 0; n < NTW; ++n) Ot[mu][n] = O::mma32(Ot[mu][n], Sb[kk][n], Bq);
                }
#pragma unroll
                for (int k2 = 0; k2 <= (mu >> 1); ++k2) {
                    const T *p = s_p + (c & 1) * L::P_BUF + (16 * mu + m) * L::LDP + 32 * k2 + 4 * gq;
                    const F8 Bp = O::ld44(p, p + 16);
#pragma unroll
                    for (int n = 0; n < NTW; ++n) Ot[mu][n] = O::mma32(Ot[mu][n], Ub[k2][n], Bp);
                }
            }
            put_rows(c, Ot);
        }

        // S <- Diag(gamma_C) S + Kbar^T U
#pragma unroll
        for (int r = 0; r < DKT; ++r) {
            const f32x4 gm = *(const f32x4 *)(s_gam + 16 * r + 4 * gq);
#pragma unroll
            for (int n = 0; n < NTW; ++n) S[r][n] *= gm;
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const T *p = s_kbt + (c & 1) * L::KBT_BUF + (16 * r + m) * L::LDK + 32 * k2 + 4 * gq;
                const F8 Af = O::ld44(p, p + 16);
#pragma unroll
                for (int n = 0; n < NTW; ++n) S[r][n] = O::mma32(S[r][n], Af, Ub[k2][n]);
            }
        }
    };

    // Rung stores and the zero test after chunk c.
    auto rungs = [&](int c) {
        const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
        if (a.interval > 0) {
            if (MODE == kModePrefill && a.ckpt_S) {
                const int64_t p = (int64_t)(c + 1) * kChunk;
                if (p <= len && (pbase + p) % a.interval == 0) {
                    const int64_t rowc = (a.ckpt_off ? a.ckpt_off[u] : 0) +
                                         (pbase + p) / a.interval - pbase / a.interval - 1;
                    store_state<DKT, NTW>(a.ckpt_S + (rowc * H + h) * DK * DV, DV, wcol, gq, m, S, false);
                }
            }
            if (MODE == kModeFixup && a.ckpt_S) {
                // rung p of this segment: the propagated incoming state plus the
                // segment's own part (sub_D), i.e. Pi_p S_in + S0_p
                const int64_t p = t0 + (int64_t)(c + 1) * kChunk;   // sequence-relative
                if (p <= t1 && p % a.interval == 0) {
                    const int64_t off = ((p / a.interval - 1) * H + h) * DK * DV;
                    store_state_add<DKT, NTW>(a.ckpt_S + off, a.ckpt_in + off, DV, wcol, gq, m, S);
                }
            }
            if (MODE == kModePackage || MODE == kModePackageM) {
                const int64_t p = t0 + (int64_t)(c + 1) * kChunk;   // sequence-relative (one sequence)
                float *dst = MB ? a.ckpt_M : a.ckpt_S;
                if (dst && p <= t1 && p % a.interval == 0) {
                    const int64_t rowc = p / a.interval - 1;
                    store_state<DKT, NTW>(dst + (rowc * H + h) * DK * LDST, LDST, wcol, gq, m, S, false);
                }
            }
        }
        // M blocks with an operator: the propagated identity at the first rung
        // of the operator's interval after the segment start, within its chunks
        if (MB && xch > 0 && xo.Pi && xo.interval > 0 && c < xch) {
            const int64_t p = t0 + (int64_t)(c + 1) * kChunk;
            if (p <= t1 && p == (t0 / xo.interval + 1) * xo.interval)
                store_state<DKT, NTW>(xo.Pi + (ux * H + h) * DK * DK, DK, wcol, gq, m, S, false);
        }
        if (R::CHECK0) {
            const bool nz = state_nonzero();
            if (lane == 0) s_flag[pw] = nz ? 1 : 0;
        }
    };

    // M blocks with an operator: the chunks after which this block's columns
    // of the propagated identity are exactly zero (c, when it vanished, or
    // the end of a whole segment), or -1: past X_chunks, or the end of a
    // first sub-segment that did not vanish.
    auto put_len = [&](int c, bool vanished) {
        if (xch > 0 && pw == 0 && lane == 0) {
            const int l = (vanished || xo.whole) && c <= xch ? c : -1;
            for (int j = cbase / 64; j < (cbase + NB) / 64; ++j)
                xo.len[(ux * H + h) * (DK / 64) + j] = l;
        }
    };

    // prologue: the producers prepare chunk 0
    __syncthreads();                                                          // BA
    __syncthreads();                                                          // BB
    for (int c = 0; c < nchunks; ++c) {
        if (R::CHECK0 && c > 0 && !(s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3])) {
            // The state after chunk c-1 is exactly zero and stays zero.
            if (MB) {
                put_len(c, true);
                if (xch > 0 && xo.Pi && xo.interval > 0) {   // Pi of a rung not reached: zero
                    const int64_t first = (t0 / xo.interval + 1) * xo.interval;
                    if (first >= t0 + (int64_t)c * kChunk && first <= t1 &&
                        first <= t0 + (int64_t)xch * kChunk)
                        store_state<DKT, NTW>(xo.Pi + (ux * H + h) * DK * DK, DK, wcol, gq, m, S, true);
                }
                if (a.interval > 0 && a.ckpt_M) {
                    const int64_t first = (t0 + (int64_t)c * kChunk) / a.interval + 1;
                    for (int64_t mm = first; mm * a.interval <= t1; ++mm)
                        store_state<DKT, NTW>(a.ckpt_M + ((mm - 1) * H + h) * DK * DK, DK, wcol, gq, m, S, true);
                }
                store_state<DKT, NTW>(package_slot(a.M_out, a.M_last, a.X_per, u, H, h, DK * DK), DK,
                                      wcol, gq, m, S, true);
            }
            copy_rungs_after(t0 + (int64_t)c * kChunk);
            return;
        }
        apply(c);
        __syncthreads();                                                      // BA
        rungs(c);
        __syncthreads();                                                      // BB
    }

    if (MODE == kModePrefill) {
        float *dst = nullptr;
        if (a.s_out_idx) {
            const int32_t slot = a.s_out_idx[u];
            if (slot >= 0 && slot < a.n_slots) dst = a.S_out + ((int64_t)slot * H + h) * DK * DV;
        } else if (a.S_out) {
            dst = a.S_out + (int64_t)(u * H + h) * DK * DV;
        }
        if (dst) store_state<DKT, NTW>(dst, DV, wcol, gq, m, S, false);
    }
    if (MODE == kModePackage || MODE == kModePackageM) {
        put_len(nchunks, false);
        if (MB)
            store_state<DKT, NTW>(package_slot(a.M_out, a.M_last, a.X_per, u, H, h, DK * DK), DK, wcol,
                                  gq, m, S, false);
        else
            store_state<DKT, NTW>(package_slot(a.S_out, a.S_last, a.X_per, u, H, h, DK * DV), DV, wcol,
                                  gq, m, S, false);
    }
}

template <int DK, int DV, int NB, bool BF, int MODE, bool MB>
__device__ __forceinline__ void engine_body(const EngineArgs &a, unsigned char *smem, const int u,
                                            const int h, const int cbase, const int64_t t0,
                                            const int64_t t1) {
    const int nchunks = (int)((t1 - t0 + kChunk - 1) / kChunk);
    // with a fix-up operator the unit was corrected by fixop_kernel unless it
    // routed the unit here (route 1: the recurrence)
    if (MODE == kModeFixup && a.X_route && a.X_route[(int64_t)u * a.H + h] == 0) return;
    if (threadIdx.x < 8) ((int *)(smem + Lds<DK, NB, BF>::o_sync))[threadIdx.x] = -1;
    __syncthreads();
    // wave index as a scalar: the role branches below are wave-uniform
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wv >= 4) {
        consumer<DK, DV, NB, BF, MODE, MB>(a, smem, u, h, cbase, t0, t1, nchunks, wv - 4);
        return;
    }
    if (MODE == kModeFixup) {   // mirror the consumers' test of the incoming state
        const int *s_flag = (const int *)smem;
        __syncthreads();
        const bool any = s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3];
        __syncthreads();
        if (!any) return;
    }
    switch (wv) {
        case 0: producer<DK, DV, NB, BF, MODE, MB, 0>(a, smem, u, h, cbase, t0, t1, nchunks); break;
        case 1: producer<DK, DV, NB, BF, MODE, MB, 1>(a, smem, u, h, cbase, t0, t1, nchunks); break;
        case 2: producer<DK, DV, NB, BF, MODE, MB, 2>(a, smem, u, h, cbase, t0, t1, nchunks); break;
        default: producer<DK, DV, NB, BF, MODE, MB, 3>(a, smem, u, h, cbase, t0, t1, nchunks); break;
    }
}

template <int DK, int DV, int NB, bool BF, int MODE>
__global__ __launch_bounds__(kThreads, 1) void chunk_engine(EngineArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int H = a.H;
    // Block -> (item, column block).  The column blocks of one item share
    // blockIdx mod 8, so they run on the same XCD and share its L2.
    const int ncb = a.ncb;
    const int bx = blockIdx.x;
    const int cb = (bx >> 3) % ncb;
    const int item = ((bx >> 3) / ncb) * 8 + (bx & 7);
    if (item >= a.n_units * H) return;
    const int pos = item / H;
    const int h = item - pos * H;
    const int u = a.order ? a.order[pos] : pos;
    const int64_t t0 = a.bounds[u], t1 = a.bounds[u + 1];
    engine_body<DK, DV, NB, BF, MODE, MODE == kModePackageM>(a, smem, u, h, cb * NB, t0, t1);
}

// Workgroups per unit of the fix-up operator (host side): about two per
// compute unit over the launch, at most one per item.  (Measured on the
// 131,072-token workload's 512 units: one workgroup per unit beats spreading
// the items, since each extra workgroup reads S_in again; with 128 units,
// three or four per unit are fastest.)
inline int fixop_spread(int64_t units, int items) {
    static std::atomic<int> cache[64];
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
        cus = cache[dev].load(std::memory_order_relaxed);
        if (cus <= 0) {
            if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
                cus <= 0)
                cus = 256;
            cache[dev].store(cus, std::memory_order_relaxed);
        }
    }
    const int64_t y = (2 * (int64_t)cus + units - 1) / units;
    return (int)(y < 1 ? 1 : y > items ? items : y);
}

// Fix-up from the operator.  Grid (n_units * H, Y), four waves per
// workgroup; the segment of x-index i * H + h is order[i] when an order is
// given, and its operator is read at i.  The unit's items are its chunks
// c < X_chunks, each adding
//     o_t += S_in^T X_t
// over the chunk's 64 rows when the operator covers them, and the four
// quarters of the rung among the corrected rows (rows 32p..32p+31 of
// Pi S_in + sub_D, Pi: the propagated identity there); workgroup y takes
// items y, y + Y, ...  Every workgroup with work loads S_in and tests it
// (zero, finite), and all take the same route decision (fixup_x_chunks);
// workgroup 0 writes it and copies the unit's other rungs when they go to
// their own buffer (they are sub_D).  Route 1 leaves the unit to the
// recurrence of the engine's fix-up launch that follows.  Each wave loads
// its value columns of S_in straight into matrix-core operand registers (the
// four waves read S_in once), with the rows of its first item and the values
// they update, so a workgroup with one item waits for memory once.  With
// n_units * H a multiple of 8 the workgroups of a unit run on one XCD and
// share S_in through its L2.
template <int DK, int DV, bool BF>
__global__ __launch_bounds__(256) void fixop_kernel(EngineArgs a) {
    using O = Ops<BF>;
    using T = typename O::T;
    using F8 = typename O::F8;
    constexpr int KS = DK / 32;        // 32-deep steps
    constexpr int CTW = DV / 16 / 4;   // value-column tiles per wave
    constexpr int NPI = DK / 32;       // quarters of the rung
    const int H = a.H;
    const int pos = blockIdx.x / H, h = blockIdx.x - pos * H;
    const int u = a.order ? a.order[pos] : pos;
    const int64_t t0 = a.bounds[u], t1 = a.bounds[u + 1];
    const int64_t unit = (int64_t)u * H + h, xunit = (int64_t)pos * H + h;
    const int y = blockIdx.y, Y = gridDim.y;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const bool copies = a.ckpt_S && a.interval > 0 && a.ckpt_S != a.ckpt_in;
    // the operator's counts decide which items have work
    bool valid = a.X && a.X_len;
    int lb[DK / 64];
    int lmax = 0;
#pragma unroll
    for (int j = 0; j < DK / 64; ++j) {
        lb[j] = valid ? a.X_len[xunit * (DK / 64) + j] : 0;
        valid = valid && lb[j] >= 0 && lb[j] <= a.X_chunks;
        lmax = lb[j] > lmax ? lb[j] : lmax;
    }
    const int64_t rows = valid ? ((int64_t)lmax * kChunk < t1 - t0 ? (int64_t)lmax * kChunk : t1 - t0) : 0;
    // the rung the operator's Pi may cover (fixup_x_chunks decides)
    const int64_t first = a.interval > 0 ? (t0 / a.interval + 1) * a.interval : 0;
    const bool pi_maybe = valid && a.ckpt_S && a.interval > 0 && a.X_Pi && lmax > 0 &&
                          first <= t1 && first < t0 + (int64_t)lmax * kChunk;
    // items: chunks 0 .. X_chunks-1, then the rung's quarters
    const int nchk = (int)((rows + kChunk - 1) / kChunk);
    auto active = [&](int it) { return it < a.X_chunks ? it < nchk : pi_maybe; };
    const int n_items = a.X_chunks + NPI;
    int it0 = y;
    while (it0 < n_items && !active(it0)) it0 += Y;
    if (it0 >= n_items && y != 0) return;

    const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
    const int n0 = w * CTW;
    F8 B[4][KS];            // chunk: rows 64c + 16q + m of X; rung: rows 32p + 16q + m of Pi
    f32x4 ov[4][CTW];       // the values the products add to
    const T *Xu = (const T *)a.X + (int64_t)pos * a.X_chunks * kChunk * H * DK;
    const float *Pi = a.X_Pi + xunit * DK * DK;
    const int64_t rung_off = a.interval > 0 ? ((first / a.interval - 1) * H + h) * DK * DV : 0;
    auto load_item = [&](int it) {
        if (it < a.X_chunks) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = kChunk * it + 16 * q + m;   // < X_chunks * 64
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)   // a block of X whose identity had vanished is zero
                    B[q][kk] = it < lb[(32 * kk) / 64]
                                   ? O::ld8(Xu + ((int64_t)r * H + h) * DK + 32 * kk + 8 * gq)
                                   : O::cvt8((const float[8]){0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f});
                const int64_t tok = t0 + r < t1 ? t0 + r : t1 - 1;
#pragma unroll
                for (int n = 0; n < CTW; ++n) {
                    const int64_t idx = (tok * H + h) * DV + 16 * (n0 + n) + 4 * gq;
                    if (BF) {
                        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                        const u32x2 wv = *(const u32x2 *)((const bf16_t *)a.o + idx);
                        ov[q][n] = f32x4{bits_f32(wv[0] << 16), bits_f32(wv[0] & 0xffff0000u),
                                         bits_f32(wv[1] << 16), bits_f32(wv[1] & 0xffff0000u)};
                    } else {
                        ov[q][n] = *(const f32x4 *)((const float *)a.o + idx);
                    }
                }
            }
        } else {
            const float *rung_in = a.ckpt_in + rung_off;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int r = 32 * (it - a.X_chunks) + 16 * q + m;
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    const f32x4 *pp = (const f32x4 *)(Pi + (int64_t)r * DK + 32 * kk + 8 * gq);
                    B[q][kk] = O::cvt44(pp[0], pp[1]);
                }
#pragma unroll
                for (int n = 0; n < CTW; ++n)
                    ov[q][n] = *(const f32x4 *)(rung_in + (int64_t)r * DV + 16 * (n0 + n) + 4 * gq);
            }
        }
    };
    // every load of the first item issued with S_in's
    const float *Sin = a.S_init + unit * DK * DV;
    float sv[CTW][KS][8];   // S_in's column 16(n0+n)+m, rows 32kk+8gq .. +7
#pragma unroll
    for (int n = 0; n < CTW; ++n)
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                sv[n][kk][j] = Sin[(32 * kk + 8 * gq + j) * DV + 16 * (n0 + n) + m];
    if (it0 < n_items) load_item(it0);
    // the incoming state: zero and finiteness tests over the four waves' columns
    bool nz = false, bad = false;
#pragma unroll
    for (int n = 0; n < CTW; ++n)
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                nz |= (f32_bits(sv[n][kk][j]) & 0x7fffffffu) != 0u;
                bad |= (f32_bits(sv[n][kk][j]) & 0x7f800000u) == 0x7f800000u;
            }
    const int fl = (__syncthreads_or(nz) ? 1 : 0) | (__syncthreads_or(bad) ? 2 : 0);
    int64_t pi_rung = -1;
    const int xl = (fl & 1) ? fixup_x_chunks<DK>(a, pos, h, t0, t1, fl, pi_rung) : 0;
    if (y == 0 && tid == 0) a.X_route[unit] = xl < 0 ? 1 : 0;
    if (xl < 0) return;
    if (y == 0 && copies) {
        for (int64_t p = first; p <= t1; p += a.interval) {
            if (p == pi_rung) continue;   // formed from Pi
            const int64_t off = ((p / a.interval - 1) * H + h) * DK * DV;
            for (int i = tid; i < DK * DV / 4; i += 256)
                ((f32x4 *)(a.ckpt_S + off))[i] = ((const f32x4 *)(a.ckpt_in + off))[i];
        }
    }
    if (!(fl & 1)) return;   // a zero incoming state leaves o_local final
    // from here xl == lmax, and pi_rung == first exactly when pi_maybe
    F8 A[CTW][KS];
#pragma unroll
    for (int n = 0; n < CTW; ++n)
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) A[n][kk] = O::cvt8(sv[n][kk]);
    for (int it = it0; it < n_items; it += Y) {
        if (!active(it)) continue;
        if (it != it0) load_item(it);
        if (it < a.X_chunks) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t tok = t0 + kChunk * it + 16 * q + m;
#pragma unroll
                for (int n = 0; n < CTW; ++n) {
                    f32x4 acc = ov[q][n];
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk) acc = O::mma32(acc, A[n][kk], B[q][kk]);
                    if (tok >= t1) continue;
                    // lane (m, gq) holds value columns 16n + 4gq .. + 3 of token tok
                    const int64_t idx = (tok * H + h) * DV + 16 * (n0 + n) + 4 * gq;
                    if (BF) *(bf16x4 *)((bf16_t *)a.o + idx) = Ops<true>::cvt4(acc);
                    else *(f32x4 *)((float *)a.o + idx) = acc;
                }
            }
        } else {
            float *rung = a.ckpt_S + rung_off;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int r = 32 * (it - a.X_chunks) + 16 * q + m;
#pragma unroll
                for (int n = 0; n < CTW; ++n) {
                    f32x4 acc = ov[q][n];
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk) acc = O::mma32(acc, A[n][kk], B[q][kk]);
                    *(f32x4 *)(rung + (int64_t)r * DV + 16 * (n0 + n) + 4 * gq) = acc;
                }
            }
        }
    }
}

// Workgroups per unit of the fix-up operator: every item on its own
// workgroup while the units leave room on the device, else fewer, each
// walking several items with S_in loaded once.
template <int DK, int DV, bool BF>
hipError_t launch_fixop_t(const EngineArgs &a, hipStream_t stream) {
    const int64_t grid = (int64_t)a.n_units * a.H;
    if (grid == 0) return hipSuccess;
    if (grid > INT32_MAX || a.X_chunks <= 0 || a.X_chunks > 4096) return hipErrorInvalidValue;
    const int items = a.X_chunks + DK / 32;
    const int Y = fixop_spread(grid, items);
    hipLaunchKernelGGL((fixop_kernel<DK, DV, BF>), dim3((unsigned)grid, (unsigned)Y), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
}

// Value blocks and M blocks of the segment packages in one grid, the M blocks
// last.  M blocks stop once M is exactly zero, a few chunks in; dispatched
// after every value block they fill the CUs that the shorter value blocks
// leave idle while the longest ones finish.
template <int DK, int DV, int NB, int NBM, bool BF>
__global__ __launch_bounds__(kThreads, 1) void package_engine(EngineArgs a, int grid_v) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int H = a.H;
    const bool mblk = (int)blockIdx.x >= grid_v;
    const int ncb = mblk ? a.ncb_m : a.ncb;
    const int bx = mblk ? (int)blockIdx.x - grid_v : (int)blockIdx.x;
    const int cb = (bx >> 3) % ncb;
    const int item = ((bx >> 3) / ncb) * 8 + (bx & 7);
    if (item >= a.n_units * H) return;
    const int pos = item / H;
    const int h = item - pos * H;
    const int u = a.order ? a.order[pos] : pos;
    const int64_t t0 = a.bounds[u], t1 = a.bounds[u + 1];
    if (mblk)
        engine_body<DK, DV, NBM, BF, kModePackageM, true>(a, smem, u, h, cb * NBM, t0, t1);
    else
        engine_body<DK, DV, NB, BF, kModePackage, false>(a, smem, u, h, cb * NB, t0, t1);
}

// Column block width of the M blocks (M has dk columns).
template <int DK, int NB> constexpr int nb_m() { return NB <= DK ? NB : DK; }

template <int DK, int DV, int NB, bool BF>
hipError_t launch_package_vm(const EngineArgs &a, hipStream_t stream) {
    constexpr int NBM = nb_m<DK, NB>();
    constexpr int lds = Lds<DK, NB, BF>::size > Lds<DK, NBM, BF>::size ? Lds<DK, NB, BF>::size
                                                                       : Lds<DK, NBM, BF>::size;
    static_assert(lds <= 160 * 1024, "LDS budget");
    auto kern = package_engine<DK, DV, NB, NBM, BF>;
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    const int64_t items8 = ((int64_t)a.n_units * a.H + 7) / 8 * 8;
    const int64_t grid_v = items8 * a.ncb, grid = grid_v + items8 * a.ncb_m;
    if (grid == 0) return hipSuccess;
    if (grid > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), lds, stream, a, (int)grid_v);
    return hipGetLastError();
}

template <int DK, int DV, int NB, bool BF, int MODE>
hipError_t launch_one(const EngineArgs &a, hipStream_t stream) {
    using L = Lds<DK, NB, BF>;
    static_assert(L::size <= 160 * 1024, "LDS budget");
    auto kern = chunk_engine<DK, DV, NB, BF, MODE>;
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, L::size);
    if (e != hipSuccess) return e;
    const int ncb = a.ncb;
    const int64_t items = (int64_t)a.n_units * a.H;
    const int64_t grid = ((items + 7) / 8) * 8 * ncb;
    if (grid == 0) return hipSuccess;
    if (grid > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), L::size, stream, a);
    return hipGetLastError();
}

template <int DK, int DV, int NB, bool BF>
hipError_t launch_modes(int mode, const EngineArgs &a, hipStream_t s) {
    switch (mode) {
        case kModePrefill: return launch_one<DK, DV, NB, BF, kModePrefill>(a, s);
        case kModePackage: return launch_one<DK, DV, NB, BF, kModePackage>(a, s);
        case kModeFixup: return launch_one<DK, DV, NB, BF, kModeFixup>(a, s);
        case kModePackageM: return launch_one<DK, DV, nb_m<DK, NB>(), BF, kModePackageM>(a, s);
        case kModePackageVM: return launch_package_vm<DK, DV, NB, BF>(a, s);
        case kModeFixOp: return launch_fixop_t<DK, DV, BF>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace
}  // namespace kda
