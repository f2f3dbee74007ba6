// kda_chunk.hip -- fused chunkwise KDA engine for gfx950 (MI355X).
//
// One workgroup of 4 wave64s walks one (unit, head, column block) through its
// chunks of 64 tokens in order, holding its slice of the recurrent state in
// MFMA accumulators (fp32) for the whole walk.  A unit is a sequence
// (prefill) or a segment (package / fix-up).  Per chunk:
//
//   load      q, k, g, beta, v rows HBM -> registers (wave w owns rows 16w..16w+15;
//             lane (m, gq) owns row 16w+m and channels 32*kk + 8*gq + 0..7)
//   prep      L2 norms (wave reductions); in-chunk cumulative log2-decay
//             (16-lane DPP scan + cross-wave totals in LDS); exponentials
//   gram      A[r,i] = beta_r sum_d k_rd k_id e^{G_rd-G_id} (i<r) and
//             P[r,i] = sum_d q_rd k_id e^{G_rd-G_id} (i<=r) on bf16 MFMA, with
//             one reference point per 16-row block so every factor stays in
//             fp32 range (diagonal blocks straight from registers)
//   UT        T_bb = (I + A_bb)^-1 for the four 16x16 diagonal blocks (fp32),
//             then block forward substitution (I + A) [W | U~] = [Diag(beta)(K*Gam) | Diag(beta)V]
//             on MFMA, each wave owning a quarter of the columns
//   state     U = U~ - W S;  O = (Q*Gam) S + P U;  S <- Diag(gamma_C) S + Kbar^T U
//             (MFMA; S is used in place as the B operand through a permuted K order)
//   store     O staged in LDS, written back with 16-byte row stores; checkpoints
//
// Modes: prefill (S from S0, outputs, checkpoints, final state), package
// (value blocks start from zero and give o_local and D; "M blocks" start from
// the identity with zero values and give M and the rung sub-packages, exiting
// exactly once M is all zeros), fix-up (the propagated incoming state with zero
// values; outputs are corrected in place; exits exactly once the state is zero).
//
// The chunkwise algebra is derived from the KDA recurrence (pegainfer PR #970
// names the (M,D) segment packages; the chunk form is the standard WY / UT
// transform of the delta rule).

#include "kda_internal.h"

namespace kda {
namespace {

typedef __bf16 bf16_t;
typedef bf16_t bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16_t bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kEps = 1e-6f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int N>
__device__ __forceinline__ float row_shr(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, x), 0x110 | N, 0xF, 0xF, true));
}
// Inclusive prefix sum across the 16 lanes of a DPP row.
__device__ __forceinline__ float scan16(float x) {
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x += row_shr<8>(x);
    return x;
}

// ---------------------------------------------------------------------------
// MFMA operand policies.  A fragment holds 8 (K=32 step) or 4 (K=16 step)
// values per lane; lane (m, gq) slot j of both operands covers the same k.
// ---------------------------------------------------------------------------
template <bool BF> struct Ops;

template <> struct Ops<true> {
    using T = bf16_t;
    using F8 = bf16x8;
    using F4 = bf16x4;
    static constexpr int PAD = 8;
    __device__ static F8 cvt8(const float *v) {
        F8 r;
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = (bf16_t)v[j];
        return r;
    }
    __device__ static F8 cvt44(f32x4 a, f32x4 b) {
        F8 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) { r[j] = (bf16_t)a[j]; r[j + 4] = (bf16_t)b[j]; }
        return r;
    }
    __device__ static F4 cvt4(f32x4 v) {
        F4 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = (bf16_t)v[j];
        return r;
    }
    __device__ static F8 ld8(const T *p) { return *(const F8 *)p; }
    __device__ static F8 ld44(const T *p0, const T *p1) {
        const F4 a = *(const F4 *)p0, b = *(const F4 *)p1;
        F8 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) { r[j] = a[j]; r[j + 4] = b[j]; }
        return r;
    }
    __device__ static F4 ld4(const T *p) { return *(const F4 *)p; }
    __device__ static void st8(T *p, const float *v) { *(F8 *)p = cvt8(v); }
    __device__ static f32x4 mma32(f32x4 c, F8 a, F8 b) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static f32x4 mma16(f32x4 c, F4 a, F4 b) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                         __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
    }
};

template <> struct Ops<false> {
    using T = float;
    struct F8 { f32x4 lo, hi; };
    using F4 = f32x4;
    static constexpr int PAD = 4;
    __device__ static F8 cvt8(const float *v) {
        F8 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) { r.lo[j] = v[j]; r.hi[j] = v[j + 4]; }
        return r;
    }
    __device__ static F8 cvt44(f32x4 a, f32x4 b) { return F8{a, b}; }
    __device__ static F4 cvt4(f32x4 v) { return v; }
    __device__ static F8 ld8(const T *p) { return F8{*(const f32x4 *)p, *(const f32x4 *)(p + 4)}; }
    __device__ static F8 ld44(const T *p0, const T *p1) {
        return F8{*(const f32x4 *)p0, *(const f32x4 *)p1};
    }
    __device__ static F4 ld4(const T *p) { return *(const f32x4 *)p; }
    __device__ static void st8(T *p, const float *v) {
        *(f32x4 *)p = f32x4{v[0], v[1], v[2], v[3]};
        *(f32x4 *)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
    __device__ static f32x4 mma32(f32x4 c, F8 a, F8 b) {
#pragma unroll
        for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[s], b.lo[s], c, 0, 0, 0);
#pragma unroll
        for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[s], b.hi[s], c, 0, 0, 0);
        return c;
    }
    __device__ static f32x4 mma16(f32x4 c, F4 a, F4 b) {
#pragma unroll
        for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
        return c;
    }
};

// Global I/O of 8 consecutive elements (16-byte aligned for bf16, 32 for fp32).
template <bool BF> struct IO;
template <> struct IO<true> {
    __device__ static void load8(const void *base, int64_t idx, float *out) {
        const uint4 raw = *(const uint4 *)((const bf16_t *)base + idx);
        const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            out[2 * j] = __builtin_bit_cast(float, w4[j] << 16);
            out[2 * j + 1] = __builtin_bit_cast(float, w4[j] & 0xffff0000u);
        }
    }
    __device__ static void store8(void *base, int64_t idx, const float *v) {
        *(bf16x8 *)((bf16_t *)base + idx) = Ops<true>::cvt8(v);
    }
};
template <> struct IO<false> {
    __device__ static void load8(const void *base, int64_t idx, float *out) {
        const float4 a = *(const float4 *)((const float *)base + idx);
        const float4 b = *(const float4 *)((const float *)base + idx + 4);
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    }
    __device__ static void store8(void *base, int64_t idx, const float *v) {
        float *p = (float *)base + idx;
        *(float4 *)p = make_float4(v[0], v[1], v[2], v[3]);
        *(float4 *)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
};

__device__ __forceinline__ void load8f(const float *p, float *out) {
    const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// ---------------------------------------------------------------------------
// LDS layout (bytes).  Row paddings shift consecutive rows by 16 bytes.
// ---------------------------------------------------------------------------
template <int DK, int NB, bool BF> struct Lds {
    using T = typename Ops<BF>::T;
    static constexpr int PAD = Ops<BF>::PAD;
    static constexpr int ES = (int)sizeof(T);
    static constexpr int LDQ = DK + PAD;        // [64][DK] row-major tiles
    static constexpr int LDR = DK + NB + PAD;   // [64][DK+NB] right-hand sides
    static constexpr int LDK = 64 + PAD;        // [DK][64] transposed Kbar
    static constexpr int LDP = 64 + PAD;        // [64][64] P and -A (off-diagonal)
    static constexpr int LDT = 16 + PAD;        // [4][16][16] diagonal inverses
    static constexpr int LDAD = 20;             // [4][16][16] fp32 diagonal A blocks
    static constexpr int LDO = NB + 4;          // [64][NB] fp32 output staging
    static constexpr int o_tot = 0;
    static constexpr int o_gam = o_tot + 4 * DK * 4;
    static constexpr int o_flag = o_gam + DK * 4;
    static constexpr int o_qbar = o_flag + 64;
    static constexpr int o_wneg = o_qbar + 64 * LDQ * ES;
    static constexpr int o_ro = o_wneg + 64 * LDQ * ES;
    static constexpr int o_kbt = o_ro + 48 * LDQ * ES;
    static constexpr int o_p = o_kbt + DK * LDK * ES;
    static constexpr int o_aoff = o_p + 64 * LDP * ES;
    static constexpr int o_td = o_aoff + 64 * LDP * ES;
    static constexpr int o_ad = o_td + 4 * 16 * LDT * ES;
    static constexpr int o_r = o_ad + 4 * 16 * LDAD * 4;
    static constexpr int r_bytes = 64 * LDR * ES;
    static constexpr int ost_bytes = 64 * LDO * 4;
    static constexpr int size = o_r + (r_bytes > ost_bytes ? r_bytes : ost_bytes);
    static_assert(o_qbar % 16 == 0 && o_ro % 16 == 0 && o_kbt % 16 == 0 && o_p % 16 == 0 &&
                  o_td % 16 == 0 && o_ad % 16 == 0 && o_r % 16 == 0, "LDS alignment");
    static_assert(size <= 160 * 1024, "LDS budget");
};

// Stores this wave's state slice (or zeros) to a [DK, ld] fp32 matrix.
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

// ---------------------------------------------------------------------------
// The engine.
// ---------------------------------------------------------------------------
template <int DK, int DV, int NB, bool BF, int MODE>
__global__ __launch_bounds__(256, 1) void chunk_engine(EngineArgs a) {
    using O = Ops<BF>;
    using T = typename O::T;
    using F8 = typename O::F8;
    using L = Lds<DK, NB, BF>;
    constexpr int KS = DK / 32;      // 32-channel steps per row
    constexpr int VS = NB / 32;      // 32-column steps of the value block
    constexpr int NBW = NB / 4;      // value columns per wave
    constexpr int NTW = NBW / 16;    // value column tiles per wave
    constexpr int DKT = DK / 16;     // state row tiles
    constexpr int WCW = DK / 4;      // W columns per wave
    constexpr int WTW = WCW / 16;    // W column tiles per wave
    constexpr int XT = WTW + NTW;    // substitution column tiles per wave
    static_assert(NTW >= 1 && WTW >= 1, "tile shape");

    extern __shared__ __align__(16) unsigned char smem[];
    float *s_tot = (float *)(smem + L::o_tot);
    float *s_gam = (float *)(smem + L::o_gam);
    int *s_flag = (int *)(smem + L::o_flag);
    T *s_qbar = (T *)(smem + L::o_qbar);
    T *s_wneg = (T *)(smem + L::o_wneg);
    T *s_ro = (T *)(smem + L::o_ro);
    T *s_kbt = (T *)(smem + L::o_kbt);
    T *s_p = (T *)(smem + L::o_p);
    T *s_aoff = (T *)(smem + L::o_aoff);
    T *s_td = (T *)(smem + L::o_td);
    float *s_ad = (float *)(smem + L::o_ad);
    T *s_r = (T *)(smem + L::o_r);
    float *s_ost = (float *)(smem + L::o_r);   // aliases s_r (dead by then)

    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, m = lane & 15, gq = lane >> 4;
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
    const int64_t len = t1 - t0;

    const bool mblk = (MODE == kModePackage) && (cb >= a.ncb_s);
    const int cbase = mblk ? (cb - a.ncb_s) * NB : cb * NB;
    const bool has_v = (MODE != kModeFixup) && !mblk;
    const bool has_o = !mblk;
    const bool check_zero = (MODE == kModeFixup) || mblk;
    const int wcol = cbase + w * NBW;          // first state column of this wave
    const int ld_state = mblk ? DK : DV;

    // ---- initial state -------------------------------------------------------
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
                    float val = 0.f;
                    if (src) val = src[(int64_t)row * DV + col];
                    if (mblk) val = (row == col) ? 1.f : 0.f;
                    S[r][n][i] = val;
                }
    }

    auto any_nonzero_wave = [&]() -> bool {
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
        const bool nz = any_nonzero_wave();
        if (lane == 0) s_flag[w] = nz ? 1 : 0;
        __syncthreads();
        const bool any = s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3];
        __syncthreads();
        if (!any) return;   // incoming state is zero: o_local is already final
    }

    const int nchunks = (int)((len + kChunk - 1) / kChunk);
    const int row = 16 * w + m;                 // this lane's row in the chunk

    for (int c = 0; c < nchunks; ++c) {
        const int64_t r0 = t0 + (int64_t)c * kChunk;
        const int nvalid = (int)((t1 - r0) < kChunk ? (t1 - r0) : kChunk);
        const bool valid = row < nvalid;
        const int64_t tok = r0 + row;

        // ---- load ------------------------------------------------------------
        float qv[KS * 8], kv[KS * 8], gv[KS * 8], vv[VS * 8];
        float bt = 0.f;
#pragma unroll
        for (int e = 0; e < KS * 8; ++e) { qv[e] = 0.f; kv[e] = 0.f; gv[e] = 0.f; }
#pragma unroll
        for (int e = 0; e < VS * 8; ++e) vv[e] = 0.f;
        if (valid) {
            const int64_t base = (tok * H + h) * DK;
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                IO<BF>::load8(a.k, base + 32 * kk + 8 * gq, &kv[8 * kk]);
                load8f(a.g + base + 32 * kk + 8 * gq, &gv[8 * kk]);
                if (has_o) IO<BF>::load8(a.q, base + 32 * kk + 8 * gq, &qv[8 * kk]);
            }
            bt = a.beta[tok * H + h];
            if (has_v) {
                const int64_t vb = (tok * H + h) * DV + cbase;
#pragma unroll
                for (int kk = 0; kk < VS; ++kk) IO<BF>::load8(a.v, vb + 32 * kk + 8 * gq, &vv[8 * kk]);
            }
        }

        // ---- L2 norms and in-block cumulative log2-decay -----------------------
        {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int e = 0; e < KS * 8; ++e) { sq += qv[e] * qv[e]; sk += kv[e] * kv[e]; }
            sq += __shfl_xor(sq, 16); sq += __shfl_xor(sq, 32);
            sk += __shfl_xor(sk, 16); sk += __shfl_xor(sk, 32);
            const float fk = a.l2norm ? rsqrtf(sk + kEps) : 1.f;
            const float fq = a.l2norm ? a.scale * rsqrtf(sq + kEps) : a.scale;
#pragma unroll
            for (int e = 0; e < KS * 8; ++e) { kv[e] *= fk; qv[e] *= fq; }
        }
#pragma unroll
        for (int e = 0; e < KS * 8; ++e) gv[e] = scan16(gv[e] * kLog2e);
        if (m == 15) {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                float *d = s_tot + w * DK + 32 * kk + 8 * gq;
                *(f32x4 *)d = f32x4{gv[8 * kk], gv[8 * kk + 1], gv[8 * kk + 2], gv[8 * kk + 3]};
                *(f32x4 *)(d + 4) = f32x4{gv[8 * kk + 4], gv[8 * kk + 5], gv[8 * kk + 6], gv[8 * kk + 7]};
            }
        }
        __syncthreads();                                                   // B1

        // ---- exponentials, LDS operand tiles, diagonal Gram blocks -------------
        F8 lhsK[KS], lhsQ[KS], rhsD[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            float tw[4][8];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float *p = s_tot + b * DK + 32 * kk + 8 * gq;
                const f32x4 lo = *(const f32x4 *)p, hi = *(const f32x4 *)(p + 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) { tw[b][j] = lo[j]; tw[b][j + 4] = hi[j]; }
            }
            float lk[8], lq[8], rd[8], qb[8], rk[8], ro[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float off = 0.f, gc = 0.f;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    if (b < w) off += tw[b][j];
                    gc += tw[b][j];
                }
                const float twj = (w == 0) ? tw[0][j] : (w == 1) ? tw[1][j] : (w == 2) ? tw[2][j] : tw[3][j];
                const float gl = gv[8 * kk + j];           // block-relative, <= 0
                const float x = gl + off;                  // chunk-relative
                const float e1 = ex2(gl), e2 = ex2(-gl), eG = ex2(x), eK = ex2(gc - x);
                const float kq = kv[8 * kk + j], qq = qv[8 * kk + j];
                lk[j] = bt * kq * e1;
                lq[j] = qq * e1;
                rd[j] = kq * e2;
                qb[j] = qq * eG;
                rk[j] = bt * kq * eG;
                ro[j] = kq * ex2(twj - gl);
                s_kbt[(32 * kk + 8 * gq + j) * L::LDK + row] = (T)(kq * eK);
                if (w == 0 && m == 0) s_gam[32 * kk + 8 * gq + j] = ex2(gc);
            }
            lhsK[kk] = O::cvt8(lk);
            lhsQ[kk] = O::cvt8(lq);
            rhsD[kk] = O::cvt8(rd);
            if (has_o) O::st8(s_qbar + row * L::LDQ + 32 * kk + 8 * gq, qb);
            O::st8(s_r + row * L::LDR + 32 * kk + 8 * gq, rk);
            if (w < 3) O::st8(s_ro + row * L::LDQ + 32 * kk + 8 * gq, ro);
        }
        if (has_v) {
#pragma unroll
            for (int kk = 0; kk < VS; ++kk) {
                float rv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) rv[j] = bt * vv[8 * kk + j];
                O::st8(s_r + row * L::LDR + DK + 32 * kk + 8 * gq, rv);
            }
        }
        f32x4 Ad = {0.f, 0.f, 0.f, 0.f}, Pd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            Ad = O::mma32(Ad, lhsK[kk], rhsD[kk]);
            if (has_o) Pd = O::mma32(Pd, lhsQ[kk], rhsD[kk]);
        }
        __syncthreads();                                                   // B2

        // ---- off-diagonal Gram blocks (b = w > a) -------------------------------
        for (int a2 = 0; a2 < w; ++a2) {
            F8 lk2[KS], lq2[KS];
            if (a2 == w - 1) {
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) { lk2[kk] = lhsK[kk]; lq2[kk] = lhsQ[kk]; }
            } else {
                // reference at the end of block a2: factor e^{G_r - rho_a2} <= 1
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    float lk[8], lq[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        float mid = 0.f;   // sum of the totals of blocks a2+1 .. w-1
                        for (int b = a2 + 1; b < w; ++b) mid += s_tot[b * DK + 32 * kk + 8 * gq + j];
                        const float f = ex2(gv[8 * kk + j] + mid);
                        lk[j] = bt * kv[8 * kk + j] * f;
                        lq[j] = qv[8 * kk + j] * f;
                    }
                    lk2[kk] = O::cvt8(lk);
                    lq2[kk] = O::cvt8(lq);
                }
            }
            f32x4 Ao = {0.f, 0.f, 0.f, 0.f}, Po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const F8 B = O::ld8(s_ro + (16 * a2 + m) * L::LDQ + 32 * kk + 8 * gq);
                Ao = O::mma32(Ao, lk2[kk], B);
                if (has_o) Po = O::mma32(Po, lq2[kk], B);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 16 * w + 4 * gq + i;
                s_aoff[rr * L::LDP + 16 * a2 + m] = (T)(-Ao[i]);
                if (has_o) s_p[rr * L::LDP + 16 * a2 + m] = (T)Po[i];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r_ = 4 * gq + i;
            s_ad[(16 * w + r_) * L::LDAD + m] = Ad[i];
            if (has_o) {
                s_p[(16 * w + r_) * L::LDP + 16 * w + m] = (T)((m <= r_) ? Pd[i] : 0.f);
                for (int a2 = w + 1; a2 < 4; ++a2) s_p[(16 * w + r_) * L::LDP + 16 * a2 + m] = (T)0.f;
            }
        }
        // T_bb = (I + A_bb)^-1 by forward substitution, one column per lane.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (gq == 0) {
            float tc[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float *arow = s_ad + (16 * w + r) * L::LDAD;
                float s = (r == m) ? 1.f : 0.f;
#pragma unroll
                for (int i = 0; i < r; ++i) s = fmaf(-arow[i], tc[i], s);
                tc[r] = s;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) s_td[(16 * w + r) * L::LDT + m] = (T)tc[r];
        }
        __syncthreads();                                                   // B3

        // ---- block forward substitution: (I + A) X = R for this wave's columns --
        f32x4 X[4][XT];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
            for (int ct = 0; ct < XT; ++ct) {
                if (ct >= WTW && !has_v) { X[b][ct] = f32x4{0.f, 0.f, 0.f, 0.f}; continue; }
                const int colR = (ct < WTW) ? (w * WCW + 16 * ct + m)
                                            : (DK + w * NBW + 16 * (ct - WTW) + m);
                f32x4 Y;
#pragma unroll
                for (int i = 0; i < 4; ++i) Y[i] = (float)s_r[(16 * b + 4 * gq + i) * L::LDR + colR];
#pragma unroll
                for (int a2 = 0; a2 < b; ++a2)
                    Y = O::mma16(Y, O::ld4(s_aoff + (16 * b + m) * L::LDP + 16 * a2 + 4 * gq),
                                 O::cvt4(X[a2][ct]));
                X[b][ct] = O::mma16(f32x4{0.f, 0.f, 0.f, 0.f},
                                    O::ld4(s_td + (16 * b + m) * L::LDT + 4 * gq), O::cvt4(Y));
            }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int ct = 0; ct < WTW; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s_wneg[(16 * b + 4 * gq + i) * L::LDQ + w * WCW + 16 * ct + m] = (T)(-X[b][ct][i]);
        __syncthreads();                                                   // B4

        // ---- state products -----------------------------------------------------
        F8 Sb[KS][NTW];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
            for (int n = 0; n < NTW; ++n) Sb[kk][n] = O::cvt44(S[2 * kk][n], S[2 * kk + 1][n]);
        f32x4 U[4][NTW];
#pragma unroll
        for (int mu = 0; mu < 4; ++mu)
#pragma unroll
            for (int n = 0; n < NTW; ++n) U[mu][n] = has_v ? X[mu][WTW + n] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mu = 0; mu < 4; ++mu)
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const T *p = s_wneg + (16 * mu + m) * L::LDQ + 32 * kk + 4 * gq;
                const F8 Af = O::ld44(p, p + 16);
#pragma unroll
                for (int n = 0; n < NTW; ++n) U[mu][n] = O::mma32(U[mu][n], Af, Sb[kk][n]);
            }
        F8 Ub[2][NTW];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
            for (int n = 0; n < NTW; ++n) Ub[k2][n] = O::cvt44(U[2 * k2][n], U[2 * k2 + 1][n]);
        f32x4 Oc[4][NTW];
        if (has_o) {
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
        }
#pragma unroll
        for (int r = 0; r < DKT; ++r) {
            const f32x4 gm = *(const f32x4 *)(s_gam + 16 * r + 4 * gq);
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
        if (has_o) {
#pragma unroll
            for (int mu = 0; mu < 4; ++mu)
#pragma unroll
                for (int n = 0; n < NTW; ++n)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        s_ost[(16 * mu + 4 * gq + i) * L::LDO + w * NBW + 16 * n + m] = Oc[mu][n][i];
        }
        if (check_zero) {
            const bool nz = any_nonzero_wave();
            if (lane == 0) s_flag[w] = nz ? 1 : 0;
        }
        __syncthreads();                                                   // B5

        // ---- outputs ---------------------------------------------------------------
        if (has_o) {
            constexpr int CG = NB / 8;
#pragma unroll
            for (int it = 0; it < (64 * CG) / 256; ++it) {
                const int idx = tid + 256 * it;
                const int rr = idx / CG, cg = idx - rr * CG;
                if (rr < nvalid) {
                    const float *src = s_ost + rr * L::LDO + 8 * cg;
                    float v8[8];
                    const f32x4 lo = *(const f32x4 *)src, hi = *(const f32x4 *)(src + 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) { v8[j] = lo[j]; v8[j + 4] = hi[j]; }
                    const int64_t gidx = ((r0 + rr) * H + h) * DV + cbase + 8 * cg;
                    if (MODE == kModeFixup) {
                        float o8[8];
                        IO<BF>::load8(a.o, gidx, o8);
#pragma unroll
                        for (int j = 0; j < 8; ++j) v8[j] += o8[j];
                    }
                    IO<BF>::store8(a.o, gidx, v8);
                }
            }
        }
        // ---- checkpoints -------------------------------------------------------------
        if (a.interval > 0) {
            if (MODE == kModePrefill && a.ckpt_S) {
                const int64_t p = (int64_t)(c + 1) * kChunk;
                if (p <= len && p % a.interval == 0) {
                    const int64_t rowc = (a.ckpt_off ? a.ckpt_off[u] : 0) + p / a.interval - 1;
                    store_state<DKT, NTW>(a.ckpt_S + (rowc * H + h) * DK * DV, DV, wcol, gq, m, S, false);
                }
            }
            if (MODE == kModePackage) {
                const int64_t p = r0 + kChunk;   // sequence-relative (one sequence)
                float *dst = mblk ? a.ckpt_M : a.ckpt_S;
                if (dst && p <= t1 && p % a.interval == 0) {
                    const int64_t rowc = p / a.interval - 1;
                    store_state<DKT, NTW>(dst + (rowc * H + h) * DK * ld_state, ld_state, wcol, gq, m, S, false);
                }
            }
        }
        if (check_zero) {
            const bool any = s_flag[0] | s_flag[1] | s_flag[2] | s_flag[3];
            if (!any) {
                if (MODE == kModePackage) {
                    // M stays exactly zero: remaining rungs and the package's M are zero.
                    if (a.interval > 0 && a.ckpt_M) {
                        const int64_t first = (r0 + kChunk) / a.interval + 1;
                        for (int64_t mm = first; mm * a.interval <= t1; ++mm)
                            store_state<DKT, NTW>(a.ckpt_M + ((mm - 1) * H + h) * DK * DK, DK, wcol, gq, m, S, true);
                    }
                    store_state<DKT, NTW>(a.M_out + (int64_t)(u * H + h) * DK * DK, DK, wcol, gq, m, S, true);
                }
                return;
            }
        }
    }

    // ---- final state ---------------------------------------------------------------
    if (MODE == kModePrefill && a.S_out)
        store_state<DKT, NTW>(a.S_out + (int64_t)(u * H + h) * DK * DV, DV, wcol, gq, m, S, false);
    if (MODE == kModePackage) {
        if (mblk) store_state<DKT, NTW>(a.M_out + (int64_t)(u * H + h) * DK * DK, DK, wcol, gq, m, S, false);
        else store_state<DKT, NTW>(a.S_out + (int64_t)(u * H + h) * DK * DV, DV, wcol, gq, m, S, false);
    }
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
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), L::size, stream, a);
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
    if (!bf16 || dk == 64) return 64;
    // Split the value columns when the grid would leave most CUs idle.
    const int64_t blocks128 = units * (mode == kModePackage ? 2 : 1);
    return blocks128 >= 256 ? 128 : 64;
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
