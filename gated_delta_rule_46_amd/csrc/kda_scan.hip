// kda_scan.hip -- (M,D) package scans, segment-path checkpoints and the
// longest-first work plan.
//
// Packages (pegainfer PR #970 "cross-process CP whale gang", whale-lane commit
// text: segments exchange KDA (M,D) packages, combined all-prefix or by a
// Blelloch prefix scan) map a segment's incoming state to S_out = M S_in + D.
// Composition, later after earlier: (Mb,Db) o (Ma,Da) = (Mb Ma, Mb Da + Db).
//
// Every product here is "out[DK x NC] = L[DK x DK] R[DK x NC] + Add" in fp32
// by one workgroup of four waves.  A zero L -- the usual case once a segment
// has forgotten its incoming state -- turns the product into a copy of Add,
// which is exact; the zero test reads L once with all loads in flight.  A
// nonzero L is multiplied on the fp32 matrix cores (v_mfma_f32_16x16x4_f32)
// with both operands read straight from L2; wave w owns output rows
// [w*DK/4, (w+1)*DK/4) and the whole product stays in accumulators until it
// is stored, so the output may overwrite an operand after a barrier.  No
// kernel here uses LDS beyond the barrier's own, so many workgroups share a
// CU and the copies run at streaming bandwidth.

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int NTH = 256;   // threads per workgroup (four waves)

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bool nonzero4(float4 x) {
    const uint32_t m = 0x7fffffffu;
    return ((__builtin_bit_cast(uint32_t, x.x) & m) | (__builtin_bit_cast(uint32_t, x.y) & m) |
            (__builtin_bit_cast(uint32_t, x.z) & m) | (__builtin_bit_cast(uint32_t, x.w) & m)) != 0u;
}

__device__ __forceinline__ bool nonfinite1(float x) {
    return (__builtin_bit_cast(uint32_t, x) & 0x7f800000u) == 0x7f800000u;
}

// Block-cooperative N-float tile held in registers (PER float4 per thread):
// every load of a tile is issued before any of its stores, so a copy costs one
// memory latency even where source and destination may alias.
template <int N> struct Tile {
    static constexpr int PER = N / 4 / NTH;
    static_assert(PER * 4 * NTH == N, "block size");
    f32x4 x[PER];
    __device__ __forceinline__ void load(const float *p) {
#pragma unroll
        for (int i = 0; i < PER; ++i) x[i] = ((const f32x4 *)p)[threadIdx.x + i * NTH];
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < PER; ++i) x[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __device__ __forceinline__ void store(float *p) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) ((f32x4 *)p)[threadIdx.x + i * NTH] = x[i];
    }
    __device__ __forceinline__ bool any_nonzero() const {
        uint32_t acc = 0u;
#pragma unroll
        for (int i = 0; i < PER; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc |= __builtin_bit_cast(uint32_t, x[i][c]) & 0x7fffffffu;
        return __syncthreads_or(acc != 0u) != 0;
    }
    // workgroup-uniform: some element is an infinity or a NaN
    __device__ __forceinline__ bool any_nonfinite() const {
        bool bad = false;
#pragma unroll
        for (int i = 0; i < PER; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) bad |= nonfinite1(x[i][c]);
        return __syncthreads_or(bad) != 0;
    }
};

// Workgroup-uniform test of N floats (N a multiple of 4 * NTH) for a nonzero
// element; every load is issued before the first is used.
template <int N>
__device__ __forceinline__ bool block_nonzero(const float *p) {
    constexpr int PER = N / 4 / NTH;
    static_assert(PER * 4 * NTH == N, "block size");
    float4 x[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) x[i] = ((const float4 *)p)[threadIdx.x + i * NTH];
    bool nz = false;
#pragma unroll
    for (int i = 0; i < PER; ++i) nz |= nonzero4(x[i]);
    return __syncthreads_or(nz) != 0;
}

// dst = src over N floats (zeros when src is null), 16-byte accesses.
template <int N>
__device__ __forceinline__ void copy_n(float *dst, const float *src) {
    constexpr int PER = N / 4 / NTH;
    static_assert(PER * 4 * NTH == N, "block size");
    float4 x[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i)
        x[i] = src ? ((const float4 *)src)[threadIdx.x + i * NTH] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < PER; ++i) ((float4 *)dst)[threadIdx.x + i * NTH] = x[i];
}

// Accumulators of one wave's rows of a DK x NC product.
template <int DK, int NC> struct Acc {
    static constexpr int RT = DK / 64;     // 16-row tiles per wave
    static constexpr int CT = NC / 16;     // 16-column tiles
    f32x4 v[RT][CT];
};

// acc = L R (L row-major DK x DK, R row-major DK x NC), fp32 MFMA.  Lane
// (n, g) of wave w holds rows w*DK/4 + 16 rt + 4 g + i of column 16 ct + n.
//
// lz / rz: the operand is exactly zero and its memory is not read (zeros are
// multiplied instead), so that a zero matrix times a non-finite operand gives
// NaN where the product would.
template <int DK, int NC>
__device__ __forceinline__ void mm_acc(const float *L, const float *R, Acc<DK, NC> &acc,
                                       bool lz = false, bool rz = false) {
    constexpr int RT = Acc<DK, NC>::RT, CT = Acc<DK, NC>::CT;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int r0 = w * (DK / 4);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc.v[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    // fully unrolled: the loads of later k-steps are issued while earlier
    // MFMAs run, which hides the L2 latency of the operand reads
#pragma unroll
    for (int k0 = 0; k0 < DK; k0 += 4) {
        float a[RT], b[CT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) a[rt] = lz ? 0.f : L[(int64_t)(r0 + 16 * rt + n) * DK + k0 + g];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) b[ct] = rz ? 0.f : R[(int64_t)(k0 + g) * NC + 16 * ct + n];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                acc.v[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[rt], b[ct], acc.v[rt][ct], 0, 0, 0);
    }
}

// out = acc + Add (Add may be null); each element is read and written by the
// lane that owns it.
template <int DK, int NC>
__device__ __forceinline__ void store_acc(const Acc<DK, NC> &acc, const float *Add, float *out) {
    constexpr int RT = Acc<DK, NC>::RT, CT = Acc<DK, NC>::CT;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int r0 = w * (DK / 4);
    if (Add) {
        float add[RT][CT][4];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    add[rt][ct][i] = Add[(int64_t)(r0 + 16 * rt + 4 * g + i) * NC + 16 * ct + n];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    out[(int64_t)(r0 + 16 * rt + 4 * g + i) * NC + 16 * ct + n] = acc.v[rt][ct][i] + add[rt][ct][i];
    } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    out[(int64_t)(r0 + 16 * rt + 4 * g + i) * NC + 16 * ct + n] = acc.v[rt][ct][i];
    }
}

// out = L R + Add.  With nz false L is exactly zero and is not read: out is
// a copy of Add, unless R holds an infinity or a NaN, in which case the
// product is formed with zeros for L (0 * inf and 0 * NaN are NaN, as in the
// product itself).  out must not alias L, R or Add.
template <int DK, int NC>
__device__ __forceinline__ void affine(const float *L, bool nz, const float *R, const float *Add,
                                       float *out) {
    if (!nz) {
        Tile<DK * NC> ta, tr;   // both loads in flight together
        ta.load(Add);
        tr.load(R);
        if (!tr.any_nonfinite()) {
            ta.store(out);
            return;
        }
    }
    Acc<DK, NC> acc;
    mm_acc<DK, NC>(L, R, acc, !nz);
    store_acc<DK, NC>(acc, Add, out);
}

// ---------------------------------------------------------------------------
// Sequential scan: one workgroup per head.  S_in[0] = S0, S_in[j+1] = M_j S_in[j] + D_j.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(NTH) void scan_seq_kernel(int H, int nseg, const float *M,
                                                       const float *D, const float *S0,
                                                       float *S_in, float *S_final) {
    const int h = blockIdx.x;
    const int64_t ss = (int64_t)DK * DV, mm = (int64_t)DK * DK;
    copy_n<DK * DV>(S_in + (int64_t)h * ss, S0 ? S0 + (int64_t)h * ss : nullptr);
    __syncthreads();
    for (int j = 0; j < nseg; ++j) {
        const float *Sj = S_in + ((int64_t)j * H + h) * ss;
        float *dst = (j + 1 < nseg) ? S_in + ((int64_t)(j + 1) * H + h) * ss : S_final + (int64_t)h * ss;
        const float *Mj = M + ((int64_t)j * H + h) * mm;
        const float *Dj = D + ((int64_t)j * H + h) * ss;
        // D_j is loaded with the zero test of M_j (one memory latency per
        // step in the usual case, where S_in[j+1] = D_j)
        Tile<DK * DV> td, ts;
        td.load(Dj);
        ts.load(Sj);
        // a zero M_j passes D_j on, unless S_in[j] holds an infinity or a NaN
        // (0 * NaN is NaN): then the product is formed
        if (!block_nonzero<DK * DK>(Mj) && !ts.any_nonfinite()) {
            td.store(dst);
        } else {
            affine<DK, DV>(Mj, true, Sj, Dj, dst);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Blelloch scan over packages in the workspace:
//   Pm [size+1][H][DK][DK], Pd [size+1][H][DK][DV], Fz [size+1][H]; slot
//   `size` keeps the total.  One workgroup per (pair, head), so each pair's
//   slots are touched by one workgroup only.  Flags per slot:
//     kFlagM    M may be nonzero; without it the slot's M is exactly zero
//               whatever its Pm memory holds (zero matrices are never
//               written, copied or read);
//     kFlagBad  M or D may hold an infinity or a NaN.
//   A product with a zero M is skipped only when the other factor is finite:
//   0 * inf and 0 * NaN are NaN, so against a flagged factor the product is
//   formed with zeros in place of the unread M.
// ---------------------------------------------------------------------------
constexpr int kFlagM = 1, kFlagBad = 2;

template <int DK, int DV>
__global__ __launch_bounds__(NTH, 1) void blel_init_kernel(int H, int nseg, const float *M,
                                                        const float *D, float *Pm, float *Pd,
                                                        int *Fz) {
    const int slot = blockIdx.x, h = blockIdx.y;
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    float *pm = Pm + ((int64_t)slot * H + h) * mm;
    float *pd = Pd + ((int64_t)slot * H + h) * dd;
    if (slot < nseg) {
        Tile<DK * DK> tm;
        Tile<DK * DV> td;
        tm.load(M + ((int64_t)slot * H + h) * mm);
        td.load(D + ((int64_t)slot * H + h) * dd);
        const bool nz = tm.any_nonzero();
        const bool bad = tm.any_nonfinite() || td.any_nonfinite();
        if (nz) tm.store(pm);
        td.store(pd);
        if (threadIdx.x == 0) Fz[slot * H + h] = (nz ? kFlagM : 0) | (bad ? kFlagBad : 0);
    } else {
        for (int e = threadIdx.x; e < DK * DK; e += NTH) pm[e] = (e / DK == e % DK) ? 1.f : 0.f;
        copy_n<DK * DV>(pd, nullptr);
        if (threadIdx.x == 0) Fz[slot * H + h] = kFlagM;
    }
}

// One combine of a level, P[later] o P[earlier] = (Ml Me, Ml De + Dl):
//   up-sweep   (down = 0): P[i] <- P[i] o P[j]
//   down-sweep (down = 1): (P[j], P[i]) <- (P[i], P[j] o P[i])
// with i = (blockIdx.x + 1) * 2 * step - 1 and j = i - step.
template <int DK, int DV>
__global__ __launch_bounds__(NTH, 1) void blel_level_kernel(int H, int step, int down, float *Pm,
                                                         float *Pd, int *Fz) {
    const int h = blockIdx.y;
    const int64_t i = (int64_t)(blockIdx.x + 1) * 2 * step - 1, j = i - step;
    const int64_t lat = down ? j : i, ear = down ? i : j;
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    float *Ml = Pm + (lat * H + h) * mm, *Dl = Pd + (lat * H + h) * dd;
    float *Me = Pm + (ear * H + h) * mm, *De = Pd + (ear * H + h) * dd;
    const int fl = Fz[lat * H + h], fe = Fz[ear * H + h];
    // exact zero tests: flags first, then the memory of a flagged later M
    const bool zl = !(fl & kFlagM) || !block_nonzero<DK * DK>(Ml);
    const bool ze = !(fe & kFlagM);
    const bool bl = fl & kFlagBad, be = fe & kFlagBad;
    // Ml Me is exactly zero when both are zero, or one is zero and the other finite
    const bool need_mm = !((zl && ze) || (zl && !be) || (ze && !bl));
    // Ml De is exactly zero when Ml is zero and De finite
    const bool need_md = !(zl && !be);
    Acc<DK, DK> am;
    Acc<DK, DV> ad;
    if (need_mm) mm_acc<DK, DK>(Ml, Me, am, zl, ze);
    if (need_md) mm_acc<DK, DV>(Ml, De, ad, zl, false);
    __syncthreads();                       // every operand read precedes the first store
    const int flags = (need_mm ? kFlagM : 0) | ((bl || be) ? kFlagBad : 0);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int r0 = w * (DK / 4);
    // each lane moves exactly the elements it owns in the accumulator layout
    if (!down) {
        // result into slot i (= later)
        if (need_mm) store_acc<DK, DK>(am, nullptr, Ml);
        if (need_md) store_acc<DK, DV>(ad, Dl, Dl);
        __syncthreads();                   // every wave has read the flags
        if (threadIdx.x == 0) Fz[i * H + h] = flags;
        return;
    }
    // down-sweep: slot j (= later) takes the old P[i] (= earlier), slot i the result
    if (!need_mm && !need_md) {
        // the usual case (Ml zero against finite factors): P[j] <- P[i],
        // P[i] <- (0, Dj); whole tiles through registers, every load before
        // any store
        if (fe & kFlagM) {
            Tile<DK * DK> t;
            t.load(Me);
            t.store(Ml);
        }
        Tile<DK * DV> a, b;
        a.load(De);
        b.load(Dl);
        a.store(Dl);
        b.store(De);
        __syncthreads();                   // every wave has read the flags
        if (threadIdx.x == 0) { Fz[j * H + h] = fe; Fz[i * H + h] = flags; }
        return;
    }
    if ((fe & kFlagM) || need_mm) {
#pragma unroll
        for (int rt = 0; rt < Acc<DK, DK>::RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < Acc<DK, DK>::CT; ++ct)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t e = (int64_t)(r0 + 16 * rt + 4 * g + q) * DK + 16 * ct + n;
                    if (fe & kFlagM) Ml[e] = Me[e];
                    if (need_mm) Me[e] = am.v[rt][ct][q];
                }
    }
#pragma unroll
    for (int rt = 0; rt < Acc<DK, DV>::RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < Acc<DK, DV>::CT; ++ct)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t e = (int64_t)(r0 + 16 * rt + 4 * g + q) * DV + 16 * ct + n;
                const float od = Dl[e];
                Dl[e] = De[e];
                De[e] = need_md ? ad.v[rt][ct][q] + od : od;
            }
    __syncthreads();                       // every wave has read the flags
    if (threadIdx.x == 0) { Fz[j * H + h] = fe; Fz[i * H + h] = flags; }
}

// After the up-sweep: slot `size` = total, slot size-1 = identity.
template <int DK, int DV>
__global__ __launch_bounds__(NTH) void blel_root_kernel(int H, int size, float *Pm, float *Pd,
                                                        int *Fz) {
    const int h = blockIdx.x;
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    float *lm = Pm + ((int64_t)(size - 1) * H + h) * mm, *ld = Pd + ((int64_t)(size - 1) * H + h) * dd;
    float *tm = Pm + ((int64_t)size * H + h) * mm, *td = Pd + ((int64_t)size * H + h) * dd;
    const int f_last = Fz[(size - 1) * H + h];
    {
        Tile<DK * DK> t;
        if (f_last & kFlagM) {
            t.load(lm);
            t.store(tm);
        }
#pragma unroll
        for (int k = 0; k < Tile<DK * DK>::PER; ++k) {
            const int64_t e = threadIdx.x + (int64_t)k * NTH;
            const int r = (int)((4 * e) / DK), c = (int)((4 * e) % DK);
            t.x[k] = f32x4{r == c ? 1.f : 0.f, r == c + 1 ? 1.f : 0.f, r == c + 2 ? 1.f : 0.f,
                           r == c + 3 ? 1.f : 0.f};
        }
        t.store(lm);
    }
    {
        Tile<DK * DV> t;
        t.load(ld);
        t.store(td);
        t.zero();
        t.store(ld);
    }
    __syncthreads();   // every wave has read the flags before they change
    if (threadIdx.x == 0) { Fz[size * H + h] = f_last; Fz[(size - 1) * H + h] = kFlagM; }
}

// S_in[j] = P[j].M S0 + P[j].D (j < nseg);  S_final = P[size].M S0 + P[size].D.
// grid (nseg+1, H).
template <int DK, int DV>
__global__ __launch_bounds__(NTH) void blel_apply_kernel(int H, int nseg, int size, const float *Pm,
                                                         const float *Pd, const int *Fz,
                                                         const float *S0, float *S_in, float *S_final) {
    const int jj = blockIdx.x, h = blockIdx.y;
    const int slot = jj < nseg ? jj : size;
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    const float *Lm = Pm + ((int64_t)slot * H + h) * mm;
    const float *Ad = Pd + ((int64_t)slot * H + h) * dd;
    float *out = jj < nseg ? S_in + ((int64_t)jj * H + h) * dd : S_final + (int64_t)h * dd;
    if (!S0) {   // a zero incoming state
        copy_n<DK * DV>(out, Ad);
        return;
    }
    const float *s0 = S0 + (int64_t)h * dd;
    const bool nz = (Fz[slot * H + h] & kFlagM) ? block_nonzero<DK * DK>(Lm) : false;
    // a zero prefix M (not read when flagged zero) passes Ad on unless S0 is
    // not finite
    affine<DK, DV>(Lm, nz, s0, Ad, out);
}

// Segment-path checkpoints: grid (rows, H).  Rung row r sits at
// p = (r+1)*interval inside segment j (seg_start[j] < p <= seg_start[j+1]):
// states[r] = sub_M[r] S_in[j] + sub_D[r].
template <int DK, int DV>
__global__ __launch_bounds__(NTH) void ckpt_kernel(int H, int nseg, const int64_t *seg_start,
                                                   int interval, const float *S_in,
                                                   const float *sub_M, const float *sub_D,
                                                   float *states) {
    const int64_t r = blockIdx.x;
    const int h = blockIdx.y;
    const int64_t p = (r + 1) * interval;
    int j = 0;
    while (j + 1 < nseg && seg_start[j + 1] < p) ++j;
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    const float *Lm = sub_M + (r * H + h) * mm;
    const float *Sj = S_in + ((int64_t)j * H + h) * dd;
    bool nz, bad;
    {   // the zero test of sub_M and the finiteness test of S_in^j, all loads in flight
        Tile<DK * DK> tl;
        Tile<DK * DV> ts;
        tl.load(Lm);
        ts.load(Sj);
        nz = tl.any_nonzero();
        bad = ts.any_nonfinite();
    }
    const float *Dr = sub_D + (r * H + h) * dd;
    float *out = states + (r * H + h) * dd;
    if (!nz && !bad) {
        copy_n<DK * DV>(out, Dr);
        return;
    }
    Acc<DK, DV> acc;
    mm_acc<DK, DV>(Lm, Sj, acc, !nz);
    store_acc<DK, DV>(acc, Dr, out);
}

// Longest-first order of up to kPlanMax sequences (rank sort on chunk counts,
// ties by index), one workgroup.
constexpr int kPlanMax = 8192;
__global__ __launch_bounds__(1024) void plan_kernel(const int64_t *cu, int n, int32_t *order) {
    __shared__ int s_len[kPlanMax];
    for (int i = threadIdx.x; i < n; i += blockDim.x)
        s_len[i] = (int)((cu[i + 1] - cu[i] + kChunk - 1) / kChunk);
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int li = s_len[i];
        int rank = 0;
        for (int j = 0; j < n; ++j) {
            const int lj = s_len[j];
            rank += (lj > li) || (lj == li && j < i);
        }
        order[rank] = i;
    }
}

// Segment starts j*L (clipped to T) of an evenly split sequence.
__global__ void bounds_kernel(int64_t *b, int nseg, int64_t L, int64_t T) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j <= nseg) b[j] = (int64_t)j * L < T ? (int64_t)j * L : T;
}

int pow2_at_least(int n) {
    int size = 1;
    while (size < n) size *= 2;
    return size;
}

template <int DK, int DV>
hipError_t scan_seq_t(int H, int nseg, const float *M, const float *D, const float *S0,
                      float *S_in, float *S_final, hipStream_t s) {
    hipLaunchKernelGGL((scan_seq_kernel<DK, DV>), dim3(H), dim3(NTH), 0, s, H, nseg, M, D, S0,
                       S_in, S_final);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t scan_blel_t(int H, int nseg, const float *M, const float *D, const float *S0,
                       float *S_in, float *S_final, void *ws, hipStream_t s) {
    const int size = pow2_at_least(nseg);
    float *Pm = (float *)ws;
    float *Pd = Pm + (int64_t)(size + 1) * H * DK * DK;
    int *Fz = (int *)(Pd + (int64_t)(size + 1) * H * DK * DV);
    hipError_t e;
    hipLaunchKernelGGL((blel_init_kernel<DK, DV>), dim3(size, H), dim3(NTH), 0, s, H, nseg, M, D, Pm,
                       Pd, Fz);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    for (int step = 1; step < size; step *= 2) {
        hipLaunchKernelGGL((blel_level_kernel<DK, DV>), dim3(size / (2 * step), H), dim3(NTH), 0,
                           s, H, step, 0, Pm, Pd, Fz);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL((blel_root_kernel<DK, DV>), dim3(H), dim3(NTH), 0, s, H, size, Pm, Pd, Fz);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    for (int step = size / 2; step >= 1; step /= 2) {
        hipLaunchKernelGGL((blel_level_kernel<DK, DV>), dim3(size / (2 * step), H), dim3(NTH), 0,
                           s, H, step, 1, Pm, Pd, Fz);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL((blel_apply_kernel<DK, DV>), dim3(nseg + 1, H), dim3(NTH), 0, s, H, nseg,
                       size, Pm, Pd, Fz, S0, S_in, S_final);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t ckpt_t(int H, int64_t T, const int64_t *seg_start, int nseg, int interval,
                  const float *S_in, const float *sub_M, const float *sub_D, float *states,
                  hipStream_t s) {
    const int64_t rows = T / interval;
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL((ckpt_kernel<DK, DV>), dim3((unsigned)rows, H), dim3(NTH), 0, s, H, nseg,
                       seg_start, interval, S_in, sub_M, sub_D, states);
    return hipGetLastError();
}

}  // namespace

size_t blelloch_workspace(int dk, int dv, int H, int nseg) {
    const int size = pow2_at_least(nseg);
    return (size_t)(size + 1) * H * ((size_t)dk * dk + (size_t)dk * dv) * sizeof(float) +
           (size_t)(size + 1) * H * sizeof(int);
}

hipError_t launch_scan_sequential(int dk, int dv, int H, int nseg, const float *M, const float *D,
                                  const float *S0, float *S_in, float *S_final, hipStream_t s) {
    if (dk == 64 && dv == 64) return scan_seq_t<64, 64>(H, nseg, M, D, S0, S_in, S_final, s);
    if (dk == 64 && dv == 128) return scan_seq_t<64, 128>(H, nseg, M, D, S0, S_in, S_final, s);
    if (dk == 128 && dv == 64) return scan_seq_t<128, 64>(H, nseg, M, D, S0, S_in, S_final, s);
    if (dk == 128 && dv == 128) return scan_seq_t<128, 128>(H, nseg, M, D, S0, S_in, S_final, s);
    return hipErrorInvalidValue;
}

hipError_t launch_scan_blelloch(int dk, int dv, int H, int nseg, const float *M, const float *D,
                                const float *S0, float *S_in, float *S_final, void *ws,
                                hipStream_t s) {
    if (dk == 64 && dv == 64) return scan_blel_t<64, 64>(H, nseg, M, D, S0, S_in, S_final, ws, s);
    if (dk == 64 && dv == 128) return scan_blel_t<64, 128>(H, nseg, M, D, S0, S_in, S_final, ws, s);
    if (dk == 128 && dv == 64) return scan_blel_t<128, 64>(H, nseg, M, D, S0, S_in, S_final, ws, s);
    if (dk == 128 && dv == 128) return scan_blel_t<128, 128>(H, nseg, M, D, S0, S_in, S_final, ws, s);
    return hipErrorInvalidValue;
}

hipError_t launch_even_bounds(int64_t *bounds, int nseg, int64_t L, int64_t T, hipStream_t s) {
    hipLaunchKernelGGL(bounds_kernel, dim3((unsigned)((nseg + 1 + 255) / 256)), dim3(256), 0, s,
                       bounds, nseg, L, T);
    return hipGetLastError();
}

hipError_t launch_ckpt_write(int dk, int dv, int H, int64_t T, const int64_t *seg_start, int nseg,
                             int interval, const float *S_in, const float *sub_M,
                             const float *sub_D, float *states, hipStream_t s) {
    if (dk == 64 && dv == 64)
        return ckpt_t<64, 64>(H, T, seg_start, nseg, interval, S_in, sub_M, sub_D, states, s);
    if (dk == 64 && dv == 128)
        return ckpt_t<64, 128>(H, T, seg_start, nseg, interval, S_in, sub_M, sub_D, states, s);
    if (dk == 128 && dv == 64)
        return ckpt_t<128, 64>(H, T, seg_start, nseg, interval, S_in, sub_M, sub_D, states, s);
    if (dk == 128 && dv == 128)
        return ckpt_t<128, 128>(H, T, seg_start, nseg, interval, S_in, sub_M, sub_D, states, s);
    return hipErrorInvalidValue;
}

hipError_t launch_plan(const int64_t *cu_seqlens, int32_t n, int32_t *order, hipStream_t s) {
    if (n <= 0 || n > kPlanMax) return hipErrorInvalidValue;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, cu_seqlens, n, order);
    return hipGetLastError();
}

}  // namespace kda
