// kda_chunk.hip -- warp-specialised chunkwise KDA engine for gfx950 (MI355X).
//
// One workgroup (8 wave64s) walks one (unit, head, column block) through its
// chunks of 64 tokens in order.  A unit is a sequence (prefill) or a segment
// (package / fix-up).  The waves split into two roles that run concurrently:
//
//   producers (waves 0-3) prepare chunk c+1: loads (prefetched one chunk
//     ahead), L2 norms, in-chunk cumulative log2-decay, exponentials, the
//     Gram matrices A and P on MFMA, the diagonal 16x16 inverses of (I + A)
//     and the block forward substitution for W;
//   consumers (waves 4-7) own a quarter of the state's columns each (fp32 MFMA
//     accumulators) and apply chunk c: the substitution for U~, then
//         U = U~ - W S,   O = (Q*Gam) S + P U,   S <- Diag(gamma_C) S + Kbar^T U.
//
// Every wave executes the same four workgroup barriers per iteration; the
// producer's and the consumer's phases sit between the same barriers:
//
//        producer (chunk c+1)                     consumer (chunk c)
//   [B4->B1] norms, decay scan, block totals     U~ by substitution, U = U~ - W S,
//                                                O = Qbar S + P U (stored to HBM),
//                                                S <- gamma S + Kbar^T U
//   [B1->B2] factors, exponentials; writes Qbar, rungs, zero test
//            Kbar^T, beta*V, R_k; diagonal Gram
//   [B2->B3] off-diagonal Gram, T_bb; writes     -
//            P, -A blocks, T_bb
//   [B3->B4] substitution; writes -W             -
//
// The consumers read every hand-off tile before B1 and the producers rewrite
// them only after B1, so one copy of each tile suffices (gamma_C is
// double-buffered by chunk parity).  Loads are prefetched one chunk ahead into
// registers: g, k and beta at the start of [B2->B3], q and v at its end.
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

#include "kda_internal.h"
#include "kda_mfma.h"

namespace kda {
namespace {

using namespace mf;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kEps = 1e-6f;
constexpr int kThreads = 512;

// Returns x unchanged, but hides its value from the optimiser.  Lane indices
// are laundered through it at the top of every phase so that LDS addresses are
// recomputed inside the phase instead of being hoisted out of the chunk loop
// (hundreds of hoisted addresses otherwise exhaust the register file).
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Compact storage of the six strictly-lower 16x16 blocks (b, a), a < b.
__host__ __device__ constexpr int aoff_idx(int b, int a) { return b * (b - 1) / 2 + a; }

template <int DK, int NB, bool BF> struct Lds {
    using T = typename Ops<BF>::T;
    static constexpr int PAD = Ops<BF>::PAD;
    static constexpr int ES = (int)sizeof(T);
    static constexpr int LDQ = DK + PAD;        // [64][DK] row-major tiles
    static constexpr int LDK = 64 + PAD;        // [DK][64] transposed Kbar
    static constexpr int LDP = 64 + PAD;        // [64][64] P
    static constexpr int LDV = NB + PAD;        // [64][NB] beta*V
    static constexpr int LDT = 16 + PAD;        // 16x16 blocks
    static constexpr int LDAD = 20;             // fp32 16x16 blocks
    static constexpr int o_flag = 0;                                  // int[16]
    static constexpr int o_gam = 64;                                  // f32 [2][DK]
    static constexpr int o_tot = o_gam + 2 * DK * 4;                  // f32 [4][DK]
    static constexpr int o_fac = o_tot + 4 * DK * 4;                  // f32 [4][4][DK]
    static constexpr int o_qbar = o_fac + 16 * DK * 4;                // hand-off
    static constexpr int o_wneg = o_qbar + 64 * LDQ * ES;             // hand-off
    static constexpr int o_kbt = o_wneg + 64 * LDQ * ES;              // hand-off
    static constexpr int o_p = o_kbt + DK * LDK * ES;                 // hand-off
    static constexpr int o_bv = o_p + 64 * LDP * ES;                  // consumer-read scratch
    static constexpr int o_aoff = o_bv + 64 * LDV * ES;               // consumer-read scratch
    static constexpr int o_td = o_aoff + 6 * 16 * LDT * ES;           // consumer-read scratch
    static constexpr int o_ad = o_td + 4 * 16 * LDT * ES;             // producer scratch
    static constexpr int o_ro = o_ad + 4 * 16 * LDAD * 4;             // producer scratch
    static constexpr int o_rk = o_ro + 48 * LDQ * ES;                 // producer scratch
    static constexpr int size = o_rk + 64 * LDQ * ES;
    static_assert(o_qbar % 16 == 0 && o_wneg % 16 == 0 && o_kbt % 16 == 0 && o_p % 16 == 0 &&
                  o_bv % 16 == 0 && o_aoff % 16 == 0 && o_td % 16 == 0 && o_ad % 16 == 0 &&
                  o_ro % 16 == 0 && o_rk % 16 == 0, "LDS alignment");
    static_assert(size <= 160 * 1024, "LDS budget");
};

// Raw rows of one chunk held in registers between the prefetch and its use.
template <bool BF, int KS, int VS> struct Raw {
    static constexpr int W8 = BF ? 4 : 8;      // 32-bit words per 8 elements
    uint32_t q[KS * W8], k[KS * W8], g[KS * 8], v[VS * W8];
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
        for (int j = 0; j < 8; ++j) out[j] = __builtin_bit_cast(float, w[j]);
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

// Block forward substitution (I + A) X = R for one 16-column tile: R rows come
// from `rhs` (row-major, leading dim ld, column col); -A off-diagonal blocks
// and the diagonal inverses T_bb come from LDS.  X in MFMA C layout.
template <bool BF, typename L>
__device__ __forceinline__ void substitute(const typename Ops<BF>::T *rhs, int ld, int col,
                                           f32x4 (&X)[4], const typename Ops<BF>::T *s_aoff,
                                           const typename Ops<BF>::T *s_td, int m, int gq) {
    using O = Ops<BF>;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        f32x4 Y;
#pragma unroll
        for (int i = 0; i < 4; ++i) Y[i] = (float)rhs[(16 * b + 4 * gq + i) * ld + col];
#pragma unroll
        for (int a2 = 0; a2 < b; ++a2)
            Y = O::mma16(Y, O::ld4(s_aoff + (aoff_idx(b, a2) * 16 + m) * L::LDT + 4 * gq),
                         O::cvt4(X[a2]));
        X[b] = O::mma16(f32x4{0.f, 0.f, 0.f, 0.f},
                        O::ld4(s_td + (16 * b + m) * L::LDT + 4 * gq), O::cvt4(Y));
    }
}

template <int DK, int DV, int NB, bool BF, int MODE, bool MB>
__device__ __forceinline__ void engine_body(const EngineArgs &a, unsigned char *smem, const int u,
                                            const int h, const int cbase, const int64_t t0,
                                            const int64_t t1) {
    using O = Ops<BF>;
    using T = typename O::T;
    using F8 = typename O::F8;
    using L = Lds<DK, NB, BF>;
    constexpr int KS = DK / 32;      // 32-channel steps of a row
    constexpr int VS = NB / 32;      // 32-column steps of the value block
    constexpr int NBW = NB / 4;      // state columns per consumer wave
    constexpr int NTW = NBW / 16;    // state column tiles per consumer wave
    constexpr int DKT = DK / 16;     // state row tiles
    constexpr int WCW = DK / 4;      // W columns per producer wave
    constexpr int WTW = WCW / 16;    // W column tiles per producer wave
    constexpr int W8 = BF ? 4 : 8;
    constexpr bool HAS_V = (MODE != kModeFixup) && !MB;
    constexpr bool HAS_O = !MB;
    constexpr bool CHECK0 = (MODE == kModeFixup) || MB;
    constexpr int LDST = MB ? DK : DV;     // leading dim of this block's global state
    static_assert(NTW >= 1 && WTW >= 1, "tile shape");

    int *s_flag = (int *)(smem + L::o_flag);
    float *s_gam = (float *)(smem + L::o_gam);
    float *s_tot = (float *)(smem + L::o_tot);
    float *s_fac = (float *)(smem + L::o_fac);
    T *s_qbar = (T *)(smem + L::o_qbar);
    T *s_wneg = (T *)(smem + L::o_wneg);
    T *s_kbt = (T *)(smem + L::o_kbt);
    T *s_p = (T *)(smem + L::o_p);
    T *s_bv = (T *)(smem + L::o_bv);
    T *s_aoff = (T *)(smem + L::o_aoff);
    T *s_td = (T *)(smem + L::o_td);
    float *s_ad = (float *)(smem + L::o_ad);
    T *s_ro = (T *)(smem + L::o_ro);
    T *s_rk = (T *)(smem + L::o_rk);

    const int tid = threadIdx.x;
    const int lane = tid & 63, m = lane & 15, gq = lane >> 4;
    // wave index as a scalar: the role branch below is wave-uniform
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = wv < 4;
    const int pw = wv & 3;                  // producer block / consumer column quarter
    const int H = a.H;
    const int64_t len = t1 - t0;
    const int nchunks = (int)((len + kChunk - 1) / kChunk);

    if (producer) {
        // =====================================================================
        // Producers: prepare chunk c+1 while the consumers apply chunk c.
        // =====================================================================
        const int prow = 16 * pw + m;       // this lane's row in the chunk
        if (MODE == kModeFixup) {           // mirror the consumers' zero test
            __syncthreads();
            const bool any = s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3];
            __syncthreads();
            if (!any) return;
        }
        Raw<BF, KS, VS> raw;
        bool raw_valid = false;
        // Loads the rows of chunk c.  A row past the end of the unit is read
        // from the unit's first row (always in bounds) and masked to zero when
        // unpacked, so the loads need no branches and no zero-fill.
        auto row_of = [&](int c, int prow_) -> int64_t {
            const int64_t r0 = t0 + (int64_t)c * kChunk;
            return (r0 + prow_) < t1 ? r0 + prow_ : t0;
        };
        // g, k and beta of chunk c (issued once the previous rows are consumed).
        auto issue_loads_gk = [&](int c) {
            const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
            const int prow = 16 * pw + m;
            raw_valid = (t0 + (int64_t)c * kChunk + prow) < t1;
            const int64_t tok = row_of(c, prow);
            const int64_t base = (tok * H + h) * DK;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                ld_words<BF>(a.k, base + 32 * kk + 8 * gq, &raw.k[W8 * kk]);
                ld_words<false>(a.g, base + 32 * kk + 8 * gq, &raw.g[8 * kk]);
            }
            raw.b = a.beta[tok * H + h];
        };
        // q and v of chunk c (needed from phase 2 on, so issued one phase later).
        auto issue_loads_qv = [&](int c) {
            const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
            const int prow = 16 * pw + m;
            const int64_t tok = row_of(c, prow);
            const int64_t base = (tok * H + h) * DK;
            if (HAS_O) {
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) ld_words<BF>(a.q, base + 32 * kk + 8 * gq, &raw.q[W8 * kk]);
            }
            if (HAS_V) {
                const int64_t vb = (tok * H + h) * DV + cbase;
#pragma unroll
                for (int kk = 0; kk < VS; ++kk) ld_words<BF>(a.v, vb + 32 * kk + 8 * gq, &raw.v[W8 * kk]);
            }
        };

        float gl[KS * 8];                   // in-block cumulative log2-decay
        float fq = 0.f, fk = 0.f, bt = 0.f;
        F8 lhsK[KS], lhsQ[KS], rhsD[KS];   // rhsD[kk] is dead after its diagonal Gram step
        f32x4 Ad, Pd;

        // [5->1]: norms and the in-block cumulative log2-decay of the rows in
        // `raw` (kept packed), block totals to LDS.
        auto phase1 = [&]() {
            const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
            const int prow = 16 * pw + m;
            (void)prow; (void)gq;
            // padded rows act as identity: k = q = v = 0, g = 0, beta = 0
            const float vmask = raw_valid ? 1.f : 0.f;
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                float x[8];
                unpack_words<BF>(&raw.k[W8 * kk], x);
#pragma unroll
                for (int j = 0; j < 8; ++j) sk += x[j] * x[j];
                unpack_words<false>(&raw.g[8 * kk], &gl[8 * kk]);
#pragma unroll
                for (int j = 0; j < 8; ++j) gl[8 * kk + j] *= vmask;
            }
            bt = raw.b * vmask;
            sk += __shfl_xor(sk, 16); sk += __shfl_xor(sk, 32);
            fk = (a.l2norm ? rsqrtf(sk + kEps) : 1.f) * vmask;
            (void)sq;
#pragma unroll
            for (int e = 0; e < KS * 8; ++e) gl[e] = scan16(gl[e] * kLog2e);
            if (m == 15) {
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    float *d = s_tot + pw * DK + 32 * kk + 8 * gq;
                    *(f32x4 *)d = f32x4{gl[8 * kk], gl[8 * kk + 1], gl[8 * kk + 2], gl[8 * kk + 3]};
                    *(f32x4 *)(d + 4) = f32x4{gl[8 * kk + 4], gl[8 * kk + 5], gl[8 * kk + 6], gl[8 * kk + 7]};
                }
            }
        };

        // [1->2]: per-channel factors (once per channel), two exponentials per
        // element, operand tiles, diagonal Gram blocks.
        auto phase2 = [&](int cp) {
            const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
            const int prow = 16 * pw + m;
            (void)prow; (void)gq;
            // Per-channel factors of block b = pw (log2 domain, all <= 1):
            //   f0 = e^{rho_{b-1}}            (Qbar, R_k from the block-relative factor)
            //   f1 = e^{G_C - rho_{b-1}}      (Kbar)
            //   f2 = e^{tot_b}                (rhs of later blocks; block 3 keeps e^{tot_2})
            //   f3 = e^{rho_{b-1} - rho_0}    (block 2: e^{tot_1}; block 3: e^{tot_1 + tot_2})
            // where rho_a is the cumulative decay at the end of block a.
            float *fac = s_fac + pw * 4 * DK;
            for (int ch = lane; ch < DK; ch += 64) {
                const float t0_ = s_tot[ch], t1_ = s_tot[DK + ch], t2_ = s_tot[2 * DK + ch], t3_ = s_tot[3 * DK + ch];
                const float off = (pw >= 1 ? t0_ : 0.f) + (pw >= 2 ? t1_ : 0.f) + (pw >= 3 ? t2_ : 0.f);
                const float gc = t0_ + t1_ + t2_ + t3_;
                const float tw = pw == 0 ? t0_ : pw == 1 ? t1_ : t2_;
                fac[ch] = ex2(off);
                fac[DK + ch] = ex2(gc - off);
                fac[2 * DK + ch] = ex2(tw);
                fac[3 * DK + ch] = ex2(pw == 2 ? t1_ : t1_ + t2_);
                if (pw == 0) s_gam[(cp & 1) * DK + ch] = ex2(gc);
            }
            if (HAS_O) {
                float sq = 0.f;
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    float x[8];
                    unpack_words<BF>(&raw.q[W8 * kk], x);
#pragma unroll
                    for (int j = 0; j < 8; ++j) sq += x[j] * x[j];
                }
                sq += __shfl_xor(sq, 16); sq += __shfl_xor(sq, 32);
                fq = (a.l2norm ? a.scale * rsqrtf(sq + kEps) : a.scale) * (raw_valid ? 1.f : 0.f);
            }
            if (HAS_V) {
#pragma unroll
                for (int kk = 0; kk < VS; ++kk) {
                    float bv[8];
                    unpack_words<BF>(&raw.v[W8 * kk], bv);
#pragma unroll
                    for (int j = 0; j < 8; ++j) bv[j] *= bt;
                    O::st8(s_bv + prow * L::LDV + 32 * kk + 8 * gq, bv);
                }
            }
            Ad = f32x4{0.f, 0.f, 0.f, 0.f};
            Pd = f32x4{0.f, 0.f, 0.f, 0.f};
            wave_sync_lds();
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const int c0 = 32 * kk + 8 * gq;
                float F0[8], F1[8], F2[8];
                {
                    const f32x4 a0 = *(const f32x4 *)(fac + c0), a1 = *(const f32x4 *)(fac + c0 + 4);
                    const f32x4 b0 = *(const f32x4 *)(fac + DK + c0), b1 = *(const f32x4 *)(fac + DK + c0 + 4);
                    const f32x4 d0 = *(const f32x4 *)(fac + 2 * DK + c0), d1 = *(const f32x4 *)(fac + 2 * DK + c0 + 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        F0[j] = a0[j]; F0[j + 4] = a1[j];
                        F1[j] = b0[j]; F1[j + 4] = b1[j];
                        F2[j] = d0[j]; F2[j + 4] = d1[j];
                    }
                }
                float e1[8], e2[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) { e1[j] = ex2(gl[8 * kk + j]); e2[j] = ex2(-gl[8 * kk + j]); }
                {   // key side: lhs (x beta) and R_k = beta K Gam; rhs, rhs of later blocks, Kbar
                    float kx[8], lk[8], rd[8], t8[8];
                    unpack_words<BF>(&raw.k[W8 * kk], kx);
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float kq = kx[j] * fk;
                        lk[j] = bt * kq * e1[j];
                        rd[j] = kq * e2[j];
                    }
                    lhsK[kk] = O::cvt8(lk);
                    rhsD[kk] = O::cvt8(rd);
#pragma unroll
                    for (int j = 0; j < 8; ++j) t8[j] = lk[j] * F0[j];
                    O::st8(s_rk + prow * L::LDQ + c0, t8);
                    if (pw < 3) {
#pragma unroll
                        for (int j = 0; j < 8; ++j) t8[j] = rd[j] * F2[j];
                        O::st8(s_ro + prow * L::LDQ + c0, t8);
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) s_kbt[(c0 + j) * L::LDK + prow] = (T)(rd[j] * F1[j]);
                }
                if (HAS_O) {   // query side: lhs and Qbar = Q Gam
                    float qx[8], lq[8], t8[8];
                    unpack_words<BF>(&raw.q[W8 * kk], qx);
#pragma unroll
                    for (int j = 0; j < 8; ++j) lq[j] = qx[j] * fq * e1[j];
                    lhsQ[kk] = O::cvt8(lq);
#pragma unroll
                    for (int j = 0; j < 8; ++j) t8[j] = lq[j] * F0[j];
                    O::st8(s_qbar + prow * L::LDQ + c0, t8);
                    Pd = O::mma32(Pd, lhsQ[kk], rhsD[kk]);
                }
                Ad = O::mma32(Ad, lhsK[kk], rhsD[kk]);
                // one 32-channel step at a time keeps the fp32 temporaries short-lived
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // [2->3]: off-diagonal Gram blocks and T_bb = (I + A_bb)^-1.
        auto phase3 = [&](int cp) {
            const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
            const int prow = 16 * pw + m;
            (void)prow; (void)gq;
            // g, k and beta of this chunk are consumed: prefetch the next chunk's
            if (cp + 1 < nchunks) issue_loads_gk(cp + 1);
            const float *fac = s_fac + pw * 4 * DK;
#pragma unroll
            for (int a2 = 0; a2 < 3; ++a2) {
                if (a2 >= pw) break;
                // blocks pw >= 2, a2 <= pw - 2: lhs referenced to rho_a2, i.e. the
                // block-relative lhs times e^{rho_{pw-1} - rho_a2} <= 1 (f3, or
                // f2 = e^{tot_2} for block 3 against block 1)
                const bool scaled = a2 < pw - 1;
                const float *fs = (pw == 3 && a2 == 1) ? fac + 2 * DK : fac + 3 * DK;
                f32x4 Ao = {0.f, 0.f, 0.f, 0.f}, P_ = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    F8 lk2 = lhsK[kk], lq2 = lhsQ[kk];
                    if (scaled) {
                        const int c0 = 32 * kk + 8 * gq;
                        float x[8], y[8];
                        O::unpack8(lhsK[kk], x);
                        if (HAS_O) O::unpack8(lhsQ[kk], y);
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const float f = fs[c0 + j];
                            x[j] *= f;
                            if (HAS_O) y[j] *= f;
                        }
                        lk2 = O::cvt8(x);
                        if (HAS_O) lq2 = O::cvt8(y);
                    }
                    const F8 B = O::ld8(s_ro + (16 * a2 + m) * L::LDQ + 32 * kk + 8 * gq);
                    Ao = O::mma32(Ao, lk2, B);
                    if (HAS_O) P_ = O::mma32(P_, lq2, B);
                }
                T *dst = s_aoff + aoff_idx(pw, a2) * 16 * L::LDT;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dst[(4 * gq + i) * L::LDT + m] = (T)(-Ao[i]);
                    if (HAS_O) s_p[(16 * pw + 4 * gq + i) * L::LDP + 16 * a2 + m] = (T)P_[i];
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (HAS_O) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 16 * pw + 4 * gq + i;
                    s_p[rr * L::LDP + 16 * pw + m] = (T)((m <= 4 * gq + i) ? Pd[i] : 0.f);
                    for (int a2 = pw + 1; a2 < 4; ++a2) s_p[rr * L::LDP + 16 * a2 + m] = (T)0.f;
                }
            }

            float *ad = s_ad + pw * 16 * L::LDAD;
#pragma unroll
            for (int i = 0; i < 4; ++i) ad[(4 * gq + i) * L::LDAD + m] = Ad[i];
            wave_sync_lds();
            if (gq == 0) {
                // column m of T_bb by forward substitution; row r+1 of A_bb is
                // read while row r is being reduced
                float tc[16];
                f32x4 nxt[4];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) nxt[q4] = *(const f32x4 *)(ad + 4 * q4);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    f32x4 cur[4];
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) cur[q4] = nxt[q4];
                    if (r < 15) {
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) nxt[q4] = *(const f32x4 *)(ad + (r + 1) * L::LDAD + 4 * q4);
                    }
                    float s = (r == m) ? 1.f : 0.f;
#pragma unroll
                    for (int i = 0; i < r; ++i) s = fmaf(-cur[i >> 2][i & 3], tc[i], s);
                    tc[r] = s;
                    __builtin_amdgcn_sched_barrier(0);
                }
                T *td = s_td + pw * 16 * L::LDT;
#pragma unroll
                for (int r = 0; r < 16; ++r) td[r * L::LDT + m] = (T)tc[r];
            }
            if (cp + 1 < nchunks) issue_loads_qv(cp + 1);
        };

        // [3->4]: substitution for this wave's W columns, written as -W.
        auto phase4 = [&]() {
            const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
            const int prow = 16 * pw + m;
            (void)prow; (void)gq;
#pragma unroll
            for (int ct = 0; ct < WTW; ++ct) {
                f32x4 X[4];
                substitute<BF, L>(s_rk, L::LDQ, pw * WCW + 16 * ct + m, X, s_aoff, s_td, m, gq);
#pragma unroll
                for (int b = 0; b < 4; ++b)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        s_wneg[(16 * b + 4 * gq + i) * L::LDQ + pw * WCW + 16 * ct + m] = (T)(-X[b][i]);
            }
        };

        // prologue: chunk 0
        if (nchunks > 0) { issue_loads_gk(0); issue_loads_qv(0); phase1(); }
        __syncthreads();                                                      // B1
        if (nchunks > 0) phase2(0);
        __syncthreads();                                                      // B2
        if (nchunks > 0) phase3(0);
        __syncthreads();                                                      // B3
        if (nchunks > 0) phase4();
        __syncthreads();                                                      // B4
        for (int c = 0; c < nchunks; ++c) {
            const bool next = c + 1 < nchunks;
            if (next) phase1();
            __syncthreads();                                                  // B1
            if (next) phase2(c + 1);
            __syncthreads();                                                  // B2
            if (CHECK0 && !(s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3])) return;
            if (next) phase3(c + 1);
            __syncthreads();                                                  // B3
            if (next) phase4();
            __syncthreads();                                                  // B4
        }
        return;
    }

    // =========================================================================
    // Consumers: wave pw owns state columns wcol .. wcol + NBW - 1.
    // =========================================================================
    const int wcol = cbase + pw * NBW;
    f32x4 S[DKT][NTW];
    {
        const float *src = nullptr;
        if (MODE == kModePrefill && a.S_init) src = a.S_init + (int64_t)(u * H + h) * DK * DV;
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
                    nz |= (__builtin_bit_cast(uint32_t, S[r][n][i]) & 0x7fffffffu) != 0u;
        return __ballot(nz) != 0ull;
    };
    if (MODE == kModeFixup) {
        // An all-zero incoming state leaves o_local final: skip the unit.
        const bool nz = state_nonzero();
        if (lane == 0) s_flag[pw] = nz ? 1 : 0;
        __syncthreads();
        const bool any = s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3];
        __syncthreads();
        if (!any) return;
    }

    f32x4 U[4][NTW];
    F8 Ub[2][NTW];

    // [5->1]: U~ = substitution on beta*V, then U = U~ - W S.
    auto phase1 = [&]() {
        const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
        const int wcol = cbase + pw * NBW + 0 * m;
        (void)wcol; (void)gq;
        f32x4 Ut[4][NTW];
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
            f32x4 X[4];
            if (HAS_V) {
                substitute<BF, L>(s_bv, L::LDV, pw * NBW + 16 * n + m, X, s_aoff, s_td, m, gq);
            } else {
#pragma unroll
                for (int b = 0; b < 4; ++b) X[b] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) Ut[b][n] = X[b];
        }
        F8 Sb[KS][NTW];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int n = 0; n < NTW; ++n) Sb[kk][n] = O::cvt44(S[2 * kk][n], S[2 * kk + 1][n]);
#pragma unroll
        for (int mu = 0; mu < 4; ++mu)
#pragma unroll
            for (int n = 0; n < NTW; ++n) U[mu][n] = Ut[mu][n];
#pragma unroll
        for (int mu = 0; mu < 4; ++mu)
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const T *p = s_wneg + (16 * mu + m) * L::LDQ + 32 * kk + 4 * gq;
                const F8 Af = O::ld44(p, p + 16);
#pragma unroll
                for (int n = 0; n < NTW; ++n) U[mu][n] = O::mma32(U[mu][n], Af, Sb[kk][n]);
            }
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int n = 0; n < NTW; ++n) Ub[k2][n] = O::cvt44(U[2 * k2][n], U[2 * k2 + 1][n]);
    };

    // [1->2]: O = Qbar S + P U, stored (fix-up: added) to HBM.
    auto phase2 = [&](int c) {
        const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
        const int wcol = cbase + pw * NBW + 0 * m;
        (void)wcol; (void)gq;
        F8 Sb[KS][NTW];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int n = 0; n < NTW; ++n) Sb[kk][n] = O::cvt44(S[2 * kk][n], S[2 * kk + 1][n]);
        f32x4 Oc[4][NTW];
#pragma unroll
        for (int mu = 0; mu < 4; ++mu)
#pragma unroll
            for (int n = 0; n < NTW; ++n) Oc[mu][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mu = 0; mu < 4; ++mu)
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const T *p = s_qbar + (16 * mu + m) * L::LDQ + 32 * kk + 4 * gq;
                const F8 Af = O::ld44(p, p + 16);
#pragma unroll
                for (int n = 0; n < NTW; ++n) Oc[mu][n] = O::mma32(Oc[mu][n], Af, Sb[kk][n]);
            }
#pragma unroll
        for (int mu = 0; mu < 4; ++mu)
#pragma unroll
            for (int k2 = 0; k2 <= (mu >> 1); ++k2) {
                const T *p = s_p + (16 * mu + m) * L::LDP + 32 * k2 + 4 * gq;
                const F8 Af = O::ld44(p, p + 16);
#pragma unroll
                for (int n = 0; n < NTW; ++n) Oc[mu][n] = O::mma32(Oc[mu][n], Af, Ub[k2][n]);
            }
        const int64_t r0 = t0 + (int64_t)c * kChunk;
#pragma unroll
        for (int mu = 0; mu < 4; ++mu)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t tok = r0 + 16 * mu + 4 * gq + i;
                if (tok < t1) {
#pragma unroll
                    for (int n = 0; n < NTW; ++n) {
                        const int64_t idx = (tok * H + h) * DV + wcol + 16 * n + m;
                        float val = Oc[mu][n][i];
                        if (BF) {
                            bf16_t *o = (bf16_t *)a.o;
                            if (MODE == kModeFixup) val += (float)o[idx];
                            o[idx] = (bf16_t)val;
                        } else {
                            float *o = (float *)a.o;
                            if (MODE == kModeFixup) val += o[idx];
                            o[idx] = val;
                        }
                    }
                }
            }
    };

    // [2->3]: S <- Diag(gamma_C) S + Kbar^T U.
    auto phase3 = [&](int c) {
        const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
        const int wcol = cbase + pw * NBW + 0 * m;
        (void)wcol; (void)gq;
        const float *gam = s_gam + (c & 1) * DK;
#pragma unroll
        for (int r = 0; r < DKT; ++r) {
            const f32x4 gm = *(const f32x4 *)(gam + 16 * r + 4 * gq);
#pragma unroll
            for (int n = 0; n < NTW; ++n) S[r][n] *= gm;
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const T *p = s_kbt + (16 * r + m) * L::LDK + 32 * k2 + 4 * gq;
                const F8 Af = O::ld44(p, p + 16);
#pragma unroll
                for (int n = 0; n < NTW; ++n) S[r][n] = O::mma32(S[r][n], Af, Ub[k2][n]);
            }
        }
    };

    // [3->4]: rung stores and the zero test after chunk c.
    auto phase4 = [&](int c) {
        const int m = opaque(lane) & 15, gq = opaque(lane) >> 4;
        const int wcol = cbase + pw * NBW + 0 * m;
        (void)wcol; (void)gq;
        if (a.interval > 0) {
            if (MODE == kModePrefill && a.ckpt_S) {
                const int64_t p = (int64_t)(c + 1) * kChunk;
                if (p <= len && p % a.interval == 0) {
                    const int64_t rowc = (a.ckpt_off ? a.ckpt_off[u] : 0) + p / a.interval - 1;
                    store_state<DKT, NTW>(a.ckpt_S + (rowc * H + h) * DK * DV, DV, wcol, gq, m, S, false);
                }
            }
            if (MODE == kModePackage) {
                const int64_t p = t0 + (int64_t)(c + 1) * kChunk;   // sequence-relative (one sequence)
                float *dst = MB ? a.ckpt_M : a.ckpt_S;
                if (dst && p <= t1 && p % a.interval == 0) {
                    const int64_t rowc = p / a.interval - 1;
                    store_state<DKT, NTW>(dst + (rowc * H + h) * DK * LDST, LDST, wcol, gq, m, S, false);
                }
            }
        }
        if (CHECK0) {
            const bool nz = state_nonzero();
            if (lane == 0) s_flag[pw] = nz ? 1 : 0;
        }
    };

    // prologue: the producers prepare chunk 0
    __syncthreads();                                                          // B1
    __syncthreads();                                                          // B2
    __syncthreads();                                                          // B3
    __syncthreads();                                                          // B4
    for (int c = 0; c < nchunks; ++c) {
        // [B4 -> B1]: every read of the hand-off tiles
        phase1();
        if (HAS_O) phase2(c);
        phase3(c);
        __syncthreads();                                                      // B1
        // [B1 -> B2]: rung stores, zero test
        phase4(c);
        __syncthreads();                                                      // B2
        if (CHECK0 && !(s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3])) {
            // The state is exactly zero and stays zero.
            if (MB) {
                if (a.interval > 0 && a.ckpt_M) {
                    const int64_t first = (t0 + (int64_t)(c + 1) * kChunk) / a.interval + 1;
                    for (int64_t mm = first; mm * a.interval <= t1; ++mm)
                        store_state<DKT, NTW>(a.ckpt_M + ((mm - 1) * H + h) * DK * DK, DK, wcol, gq, m, S, true);
                }
                store_state<DKT, NTW>(a.M_out + (int64_t)(u * H + h) * DK * DK, DK, wcol, gq, m, S, true);
            }
            return;
        }
        __syncthreads();                                                      // B3
        __syncthreads();                                                      // B4
    }

    if (MODE == kModePrefill && a.S_out)
        store_state<DKT, NTW>(a.S_out + (int64_t)(u * H + h) * DK * DV, DV, wcol, gq, m, S, false);
    if (MODE == kModePackage) {
        if (MB) store_state<DKT, NTW>(a.M_out + (int64_t)(u * H + h) * DK * DK, DK, wcol, gq, m, S, false);
        else store_state<DKT, NTW>(a.S_out + (int64_t)(u * H + h) * DK * DV, DV, wcol, gq, m, S, false);
    }
}

template <int DK, int DV, int NB, bool BF, int MODE>
__global__ __launch_bounds__(kThreads, 1) void chunk_engine(EngineArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int H = a.H;
    // Block -> (item, column block).  The column blocks of one item share
    // blockIdx mod 8, so they run on the same XCD and share its L2.
    const int ncb = a.ncb_s + a.ncb_m;
    const int bx = blockIdx.x;
    const int cb = (bx >> 3) % ncb;
    const int item = ((bx >> 3) / ncb) * 8 + (bx & 7);
    if (item >= a.n_units * H) return;
    const int pos = item / H;
    const int h = item - pos * H;
    const int u = a.order ? a.order[pos] : pos;
    const int64_t t0 = a.bounds[u], t1 = a.bounds[u + 1];
    if (MODE == kModePackage && cb >= a.ncb_s)
        engine_body<DK, DV, NB, BF, MODE, true>(a, smem, u, h, (cb - a.ncb_s) * NB, t0, t1);
    else
        engine_body<DK, DV, NB, BF, MODE, false>(a, smem, u, h, cb * NB, t0, t1);
}

template <int DK, int DV, int NB, bool BF, int MODE>
hipError_t launch_one(const EngineArgs &a, hipStream_t stream) {
    using L = Lds<DK, NB, BF>;
    auto kern = chunk_engine<DK, DV, NB, BF, MODE>;
    hipError_t e = hipFuncSetAttribute((const void *)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, L::size);
    if (e != hipSuccess) return e;
    const int ncb = a.ncb_s + a.ncb_m;
    const int64_t items = (int64_t)a.n_units * a.H;
    const int64_t grid = ((items + 7) / 8) * 8 * ncb;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), L::size, stream, a);
    return hipGetLastError();
}

template <int DK, int DV, int NB, bool BF>
hipError_t launch_modes(int mode, const EngineArgs &a, hipStream_t s) {
    switch (mode) {
        case kModePrefill: return launch_one<DK, DV, NB, BF, kModePrefill>(a, s);
        case kModePackage: return launch_one<DK, DV, NB, BF, kModePackage>(a, s);
        case kModeFixup: return launch_one<DK, DV, NB, BF, kModeFixup>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool engine_supported(bool bf16, int dk, int dv, int nb) {
    if (dk != dv) return false;
    if (bf16) return (dk == 64 && nb == 64) || (dk == 128 && (nb == 64 || nb == 128));
    return dk == 64 && nb == 64;
}

int engine_pick_nb(bool bf16, int dk, int dv, int64_t units, int mode) {
    (void)dv;
    (void)mode;
    if (!bf16 || dk == 64) return 64;
    // Split the value columns when the grid would leave most CUs idle.
    return units >= 256 ? 128 : 64;
}

hipError_t launch_engine(int mode, bool bf16, int dk, int dv, int nb, const EngineArgs &a,
                         hipStream_t s) {
    if (!engine_supported(bf16, dk, dv, nb)) return hipErrorInvalidValue;
    if (bf16) {
        if (dk == 64) return launch_modes<64, 64, 64, true>(mode, a, s);
        if (nb == 128) return launch_modes<128, 128, 128, true>(mode, a, s);
        return launch_modes<128, 128, 64, true>(mode, a, s);
    }
    return launch_modes<64, 64, 64, false>(mode, a, s);
}

}  // namespace kda
