// kda_scan.hip -- (M,D) package scans, segment-path checkpoints and the
// longest-first work plan.
//
// Packages (pegainfer PR #970 "cross-process CP whale gang", whale-lane commit
// text: segments exchange KDA (M,D) packages, combined all-prefix or by a
// Blelloch prefix scan) map a segment's incoming state to S_out = M S_in + D.
// Composition, later after earlier: (Mb,Db) o (Ma,Da) = (Mb Ma, Mb Da + Db).
//
// Every product here is "out[DK x NC] = L[DK x DK] R[DK x NC] + Add" in fp32.
// A zero L -- the usual case once a segment has forgotten its incoming state
// -- turns the product into a copy of Add, which is exact; the zero test
// reads L once with all loads in flight.  In the Blelloch and split kernels a
// nonzero L is multiplied by one workgroup of four waves on the fp32 matrix
// cores (v_mfma_f32_16x16x4_f32) with both operands read straight from L2;
// wave w owns output rows [w*DK/4, (w+1)*DK/4) and the whole product stays in
// accumulators until it is stored, so the output may overwrite an operand
// after a barrier.  The sequential scan splits a head's columns over several
// workgroups and forms its products on the VALU (see there).  The kernels use
// little LDS, so many workgroups share a CU and the copies run at streaming
// bandwidth.

#include <algorithm>
#include <atomic>
#include <mutex>

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int NTH = 256;   // threads per workgroup (four waves)

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bool nonzero4(float4 x) {
    const uint32_t m = 0x7fffffffu;
    return ((f32_bits(x.x) & m) | (f32_bits(x.y) & m) | (f32_bits(x.z) & m) | (f32_bits(x.w) & m)) != 0u;
}

__device__ __forceinline__ bool nonfinite1(float x) {
    return (f32_bits(x) & 0x7f800000u) == 0x7f800000u;
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
            for (int c = 0; c < 4; ++c) acc |= f32_bits(x[i][c]) & 0x7fffffffu;
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
__device__ __forceinline__ void copy_n(float *dst, const float *src, int tid = threadIdx.x) {
    constexpr int PER = N / 4 / NTH;
    static_assert(PER * 4 * NTH == N, "block size");
    float4 x[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i)
        x[i] = src ? ((const float4 *)src)[tid + i * NTH] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < PER; ++i) ((float4 *)dst)[tid + i * NTH] = x[i];
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
// lk / rk: kMem reads the operand; kZero multiplies zeros and kIdent the
// identity without reading it, so that a zero or identity matrix times a
// non-finite operand gives NaN where the IEEE product would.
constexpr int kMem = 0, kZero = 1, kIdent = 2;
// w: the wave's index among the four that share the product (default: the
// workgroup's own wave index, four-wave workgroups).
template <int DK, int NC>
__device__ __forceinline__ void mm_acc(const float *L, const float *R, Acc<DK, NC> &acc,
                                       int lk = kMem, int rk = kMem, int w = -1) {
    constexpr int RT = Acc<DK, NC>::RT, CT = Acc<DK, NC>::CT;
    const int lane = opaque(threadIdx.x & 63);
    if (w < 0) w = threadIdx.x >> 6;
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
        for (int rt = 0; rt < RT; ++rt) {
            const int row = r0 + 16 * rt + n, col = k0 + g;
            a[rt] = lk == kMem ? L[(int64_t)row * DK + col] : (lk == kIdent && row == col) ? 1.f : 0.f;
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int row = k0 + g, col = 16 * ct + n;
            b[ct] = rk == kMem ? R[(int64_t)row * NC + col] : (rk == kIdent && row == col) ? 1.f : 0.f;
        }
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
__device__ __forceinline__ void store_acc(const Acc<DK, NC> &acc, const float *Add, float *out,
                                          int w = -1) {
    constexpr int RT = Acc<DK, NC>::RT, CT = Acc<DK, NC>::CT;
    const int lane = threadIdx.x & 63;
    if (w < 0) w = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int r0 = w * (DK / 4);
    if (Add) {
        // one 16-row tile at a time: its loads in flight together, and half
        // the registers of loading all of Add first
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            float add[CT][4];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    add[ct][i] = Add[(int64_t)(r0 + 16 * rt + 4 * g + i) * NC + 16 * ct + n];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    out[(int64_t)(r0 + 16 * rt + 4 * g + i) * NC + 16 * ct + n] = acc.v[rt][ct][i] + add[ct][i];
        }
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

// ---------------------------------------------------------------------------
// Sequential scan: S_in[0] = S0, S_in[j+1] = M_j S_in[j] + D_j.
//
// Column c of S_in[j+1] depends only on column c of S_in[j] (and all of M_j),
// so a head's value columns are split over SEQ_P = DV / 16 workgroups that
// never wait for each other; with H a multiple of 8 the workgroups of one
// head share the XCD of blockIdx mod 8 (and its L2, where M_j is read once
// from HBM).  Each
// workgroup keeps its 16 columns of the running state in registers and walks
// the packages in batches of SEQ_NB: the loads of a batch (all of M_j for the
// zero test, its own columns of D_j) are issued together, then each step is
// either a copy of D_j -- when M_j is exactly zero and the state's columns
// are finite, which is the product's exact value -- or the product, formed
// in fp32 on the VALU from the state staged in LDS (0 * inf and 0 * NaN
// spread over a column as the product would).
// ---------------------------------------------------------------------------
constexpr int SEQ_CW = 16;   // value columns per workgroup
constexpr int SEQ_NB = 8;    // packages per batch

__device__ __forceinline__ bool nonfinite4(f32x4 x) {
    return nonfinite1(x[0]) | nonfinite1(x[1]) | nonfinite1(x[2]) | nonfinite1(x[3]);
}

// Whether each package's M has a nonzero element (grid (nseg, H)): one
// workgroup per M, so the scan's workgroups need not read M to test it.
template <int DK>
__global__ __launch_bounds__(NTH) void seq_flags_kernel(int H, const float *M, int *nz) {
    constexpr int PM = DK * DK / 4 / NTH;
    const int j = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    const f32x4 *Mj = (const f32x4 *)(M + ((int64_t)j * H + h) * DK * DK);
    f32x4 a[PM];
#pragma unroll
    for (int i = 0; i < PM; ++i) a[i] = Mj[t + i * NTH];
    uint32_t acc = 0u;
#pragma unroll
    for (int i = 0; i < PM; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc |= f32_bits(a[i][c]) & 0x7fffffffu;
    const int f = __syncthreads_or(acc != 0u) ? 1 : 0;
    if (t == 0) nz[j * H + h] = f;
}

// mz_flags (nullable): package j of head h has a nonzero M exactly when
// mz_flags[j * H + h] != 0 (seq_flags_kernel); without them every workgroup
// tests each M itself.
template <int DK, int DV>
__global__ __launch_bounds__(NTH) void scan_seq_kernel(int H, int nseg, const float *M,
                                                       const float *D, const float *S0,
                                                       float *S_in, float *S_final,
                                                       const int *mz_flags) {
    constexpr int P = DV / SEQ_CW;                 // workgroups per head
    constexpr int PS = DK * SEQ_CW / 4 / NTH;      // float4 of the state's columns per thread
    constexpr int PM = DK * DK / 4 / NTH;          // float4 of an M per thread (zero test)
    static_assert(PS >= 1 && PS * 4 * NTH == DK * SEQ_CW && PM * 4 * NTH == DK * DK, "shape");
    __shared__ f32x4 s_S[DK * SEQ_CW / 4];         // state columns for a product
    __shared__ unsigned s_fl[2];
    // blocks in groups of up to 8 heads x P: head h's workgroups are the
    // blocks of the group congruent to h mod (heads in the group)
    int h, wp;
    {
        const int b = blockIdx.x, g = b / (8 * P), w = b - g * 8 * P;
        const int hn = H - 8 * g < 8 ? H - 8 * g : 8;
        h = 8 * g + w % hn;
        wp = w / hn;
    }
    const int t = threadIdx.x, q = t & 3;
    const int64_t ss = (int64_t)DK * DV, mm = (int64_t)DK * DK;
    // element offset of this thread's i-th float4 inside a state
    auto eoff = [&](int i) -> int64_t {
        return (int64_t)((t + i * NTH) >> 2) * DV + wp * SEQ_CW + 4 * q;
    };
    auto st_ptr = [&](int j) -> float * {   // S_in[j]; j = nseg: S_final
        return j < nseg ? S_in + ((int64_t)j * H + h) * ss : S_final + (int64_t)h * ss;
    };
    // running state S_in[j] (this workgroup's columns) and whether it is finite
    f32x4 cur[PS];
    bool bad = false;
#pragma unroll
    for (int i = 0; i < PS; ++i) {
        cur[i] = S0 ? *(const f32x4 *)(S0 + (int64_t)h * ss + eoff(i)) : f32x4{0.f, 0.f, 0.f, 0.f};
        bad |= nonfinite4(cur[i]);
        *(f32x4 *)(st_ptr(0) + eoff(i)) = cur[i];
    }
    bool fin = !__syncthreads_or(bad);
    for (int j0 = 0; j0 < nseg; j0 += SEQ_NB) {
        // bit jj of mz: M_{j0+jj} has a nonzero element; of db: this
        // workgroup's columns of D_{j0+jj} hold an infinity or a NaN
        f32x4 dr[SEQ_NB][PS];
        unsigned mz = 0u, db = 0u;
#pragma unroll
        for (int jj = 0; jj < SEQ_NB; ++jj) {
            const int j = j0 + jj;
            if (j >= nseg) break;
            const float *Dj = D + ((int64_t)j * H + h) * ss;
            const f32x4 *Mj = (const f32x4 *)(M + ((int64_t)j * H + h) * mm);
            uint32_t acc = 0u;
            bool b2 = false;
#pragma unroll
            for (int i = 0; i < PS; ++i) {
                dr[jj][i] = *(const f32x4 *)(Dj + eoff(i));
                b2 |= nonfinite4(dr[jj][i]);
            }
            if (mz_flags) {
                acc = mz_flags[j * H + h] != 0 ? 1u : 0u;
            } else {
#pragma unroll
                for (int i = 0; i < PM; ++i) {
                    const f32x4 x = Mj[t + i * NTH];
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc |= f32_bits(x[c]) & 0x7fffffffu;
                }
            }
            mz |= (unsigned)(acc != 0u) << jj;
            db |= (unsigned)b2 << jj;
        }
        if (t == 0) s_fl[0] = s_fl[1] = 0u;
        __syncthreads();
        if (mz) atomicOr(&s_fl[0], mz);
        if (db) atomicOr(&s_fl[1], db);
        __syncthreads();
        mz = s_fl[0];
        db = s_fl[1];
#pragma unroll
        for (int jj = 0; jj < SEQ_NB; ++jj) {
            const int j = j0 + jj;
            if (j >= nseg) break;
            if (!((mz >> jj) & 1u) && fin) {   // S_in[j+1] = D_j exactly
#pragma unroll
                for (int i = 0; i < PS; ++i) cur[i] = dr[jj][i];
                fin = !((db >> jj) & 1u);
            } else {   // S_in[j+1] = M_j S_in[j] + D_j, k ascending in fp32
                __syncthreads();   // the previous product has read s_S
#pragma unroll
                for (int i = 0; i < PS; ++i) s_S[t + i * NTH] = cur[i];
                __syncthreads();
                const float *Mj = M + ((int64_t)j * H + h) * mm;
                f32x4 acc[PS];
#pragma unroll
                for (int i = 0; i < PS; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
                for (int k = 0; k < DK; k += 4) {
                    f32x4 mr[PS], sk[4];
#pragma unroll
                    for (int i = 0; i < PS; ++i)
                        mr[i] = *(const f32x4 *)(Mj + (int64_t)((t + i * NTH) >> 2) * DK + k);
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) sk[kk] = s_S[(k + kk) * (SEQ_CW / 4) + q];
#pragma unroll
                    for (int i = 0; i < PS; ++i)
#pragma unroll
                        for (int kk = 0; kk < 4; ++kk) acc[i] += mr[i][kk] * sk[kk];
                }
                bool b2 = false;
#pragma unroll
                for (int i = 0; i < PS; ++i) {
                    cur[i] = acc[i] + dr[jj][i];
                    b2 |= nonfinite4(cur[i]);
                }
                fin = !__syncthreads_or(b2);
            }
#pragma unroll
            for (int i = 0; i < PS; ++i) *(f32x4 *)(st_ptr(j + 1) + eoff(i)) = cur[i];
        }
        __syncthreads();   // s_fl is rewritten by the next batch
    }
}

// ---------------------------------------------------------------------------
// Blelloch scan over packages (exclusive up-sweep / down-sweep over the
// composition, identity-padded to a power of two) in two launches:
//
//   blel_flags_kernel  grid (nseg + 1, H): per package, whether M is exactly
//                      zero and whether M or D holds an infinity or a NaN;
//                      block nseg tests S0;
//   blel_kernel        grid (H, P), P workgroups of four waves per head (two
//                      fit on a CU): the tree on buffer ids, then the outputs
//                      S_in[j] = Pre_j.M S0 + Pre_j.D and S_final = Total.M S0
//                      + Total.D, output j on workgroup j mod P.
//
// Slots hold buffer ids, not matrices: an id names a caller package, a fresh
// workspace buffer, the zero matrix or the identity.  Wave 0 replays the tree
// on the ids -- in registers, one slot per lane, when it has at most 64 slots,
// else in LDS one level at a time (a wave's LDS accesses complete in order, so
// either way without barriers) -- and lists the compositions that really
// multiply; only those write a fresh buffer.  The head's workgroups share each
// level's list out (a composition's M product, then its D product or sum, fp32
// MFMA) and meet after every level that formed one (head_barrier).  Every
// workgroup replays the same decisions.  With a zero M in every package (the
// configs' gates) nothing is multiplied and no workgroup waits for another.
//
// A product with a zero factor is formed only when the other factor may hold
// an infinity or a NaN (0 * inf and 0 * NaN are NaN), with zeros in place of
// the zero factor; otherwise it is exactly zero and skipped.
// ---------------------------------------------------------------------------
constexpr int kIdZero = -1, kIdIdent = -2;
constexpr int kMaxSize = 1 << 12;   // padded package count (slot kMaxSize + 1 parks a slot)

struct BlelWs {
    float *Mw, *Dw;                // fresh buffers [2 * size][H][dk][dk] and [2 * size][H][dk][dv]
    unsigned long long *bar;       // [2][H]: arrivals at the head's barriers (plain, fenced)
    int *fz, *fb;                  // [nseg][H]: M nonzero, M or D not finite
    int *s0bad;                    // [H]
};

// dst = a + b over N floats by NTH threads (tid = 0..NTH-1), every load
// before any store.
template <int N>
__device__ __forceinline__ void add_n(float *dst, const float *a, const float *b,
                                      int tid = threadIdx.x) {
    constexpr int PER = N / 4 / NTH;
    static_assert(PER * 4 * NTH == N, "block size");
    f32x4 x[PER], y[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        x[i] = ((const f32x4 *)a)[tid + i * NTH];
        y[i] = ((const f32x4 *)b)[tid + i * NTH];
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) ((f32x4 *)dst)[tid + i * NTH] = x[i] + y[i];
}

// Four waves per workgroup; the slot ids and the level's list are 16-bit, so
// that two workgroups fit in a CU's LDS.
constexpr int NTH_TREE = NTH;

// XCD (accelerator complex die) the wave runs on: hardware register
// HW_REG_XCC_ID (20), bits [3:0].
__device__ __forceinline__ int xcc_id() {
    return __builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)) & 15;
}

// Barrier counters tagged with the launch that uses them: the high word of a
// counter holds that launch's epoch, the low word the arrivals in it.  A
// counter that holds another epoch (left by an earlier launch, or never
// written) counts as zero and is restarted by the first arrival, so nothing
// has to clear the counters between launches.
__device__ __forceinline__ void arrive(unsigned long long *cnt, uint32_t epoch, uint32_t add,
                                       int order) {
    unsigned long long old = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int it = 0; it < (1 << 20); ++it) {
        const unsigned long long nw = (uint32_t)(old >> 32) == epoch
                                          ? old + add
                                          : ((unsigned long long)epoch << 32) | add;
        if (order == __ATOMIC_RELEASE) {
            if (__hip_atomic_compare_exchange_strong(cnt, &old, nw, __ATOMIC_RELEASE,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                return;
        } else if (__hip_atomic_compare_exchange_strong(cnt, &old, nw, __ATOMIC_RELAXED,
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
            return;
        }
    }
}
__device__ __forceinline__ uint32_t arrivals(const unsigned long long *cnt, uint32_t epoch,
                                             int order) {
    const unsigned long long v = order == __ATOMIC_ACQUIRE
        ? __hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT)
        : __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return (uint32_t)(v >> 32) == epoch ? (uint32_t)v : 0u;
}

// The P workgroups of one head meet here.  Workgroups are dispatched to the
// eight XCDs round-robin by linear index, and in the grid (H, P) with H a
// multiple of 8 the P workgroups of a head then run on one XCD, whose L2 they
// share: a workgroup waits for its own stores (they reach L2), arrives at the
// head's counter and waits for the other arrivals; what the others stored is
// then read through that L2.  At the first barrier every workgroup also
// reports whether it runs on a different XCD than the head's first workgroup
// would by that dispatch (bit 16 of the count: always so for some workgroups
// when H is not a multiple of 8).  If one does, every barrier of that head
// also writes the L2 back and invalidates it (device fences) around a second
// count, which makes the stores visible across XCDs.  The waits are bounded
// (2^20 polls each), so a broken count shows as wrong values, not as a hang;
// every workgroup of the launch fits on the device at once (at most half of
// what it holds), so the waits end.
__device__ __forceinline__ void head_barrier(unsigned long long *cnt, unsigned long long *cnt2,
                                             int P, int round, bool first, bool misplaced,
                                             int &mixed, uint32_t epoch) {
    __shared__ int s_mixed;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        arrive(cnt, epoch, (first && misplaced) ? 1u + (1u << 16) : 1u, __ATOMIC_RELAXED);
        uint32_t v = 0;
        for (int it = 0; it < (1 << 20); ++it) {
            v = arrivals(cnt, epoch, __ATOMIC_RELAXED);
            if ((int)(v & 0xffffu) >= P * round) break;
            __builtin_amdgcn_s_sleep(2);
        }
        if (first) s_mixed = (v >> 16) != 0;
    }
    __syncthreads();
    if (first) mixed = s_mixed;
    if (mixed) {
        if (threadIdx.x == 0) {
            __threadfence();
            arrive(cnt2, epoch, 1u, __ATOMIC_RELEASE);
            for (int it = 0; it < (1 << 20); ++it) {
                if ((int)arrivals(cnt2, epoch, __ATOMIC_ACQUIRE) >= P * round) break;
                __builtin_amdgcn_s_sleep(2);
            }
            __threadfence();
        }
        __syncthreads();
    }
    asm volatile("" ::: "memory");
}

// A flag another workgroup stored before a barrier, read past the vector L1.
__device__ __forceinline__ int load_flag(const int *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Flags of one unit per workgroup, grid (nseg + 1, H): package u (M exactly
// zero or not; M or D holding an infinity or a NaN), or S0 for u = nseg.
template <int DK, int DV>
__global__ __launch_bounds__(NTH) void blel_flags_kernel(int H, int nseg, const float *M,
                                                         const float *D, const float *S0,
                                                         BlelWs w) {
    constexpr int PM = DK * DK / 4 / NTH, PD = DK * DV / 4 / NTH;
    const int u = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    bool nz = false, bad = false;
    if (u < nseg) {
        const f32x4 *Mu = (const f32x4 *)(M + ((int64_t)u * H + h) * mm);
        const f32x4 *Du = (const f32x4 *)(D + ((int64_t)u * H + h) * dd);
        f32x4 a[PM], b[PD];
#pragma unroll
        for (int i = 0; i < PM; ++i) a[i] = Mu[t + i * NTH];
#pragma unroll
        for (int i = 0; i < PD; ++i) b[i] = Du[t + i * NTH];
        uint32_t acc = 0u;
#pragma unroll
        for (int i = 0; i < PM; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                acc |= f32_bits(a[i][c]) & 0x7fffffffu;
                bad |= nonfinite1(a[i][c]);
            }
#pragma unroll
        for (int i = 0; i < PD; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) bad |= nonfinite1(b[i][c]);
        nz = acc != 0u;
    } else if (S0) {
        const f32x4 *Su = (const f32x4 *)(S0 + (int64_t)h * dd);
        f32x4 b[PD];
#pragma unroll
        for (int i = 0; i < PD; ++i) b[i] = Su[t + i * NTH];
#pragma unroll
        for (int i = 0; i < PD; ++i)
#pragma unroll
            for (int c = 0; c < 4; ++c) bad |= nonfinite1(b[i][c]);
    }
    const int fnz = __syncthreads_or(nz) ? 1 : 0, fbad = __syncthreads_or(bad) ? 1 : 0;
    if (t == 0) {
        if (u < nseg) {
            w.fz[u * H + h] = fnz;
            w.fb[u * H + h] = fbad;
        } else {
            w.s0bad[h] = fbad;
        }
    }
}

// r <- l o e = (Ml Me, Ml De + Dl) on ids: the ids r takes, the products it
// needs (M: mprod; D: dkind 1 a sum, 2 a product) and the operand kinds.  A
// zero or identity factor is used as such only against finite values: under
// IEEE arithmetic 0 * inf is NaN and I X spreads an inf or a NaN of X over
// its column, so against a non-finite factor the product is formed (with the
// zero or identity substituted).
struct Decision {
    int rm, rd, mprod, dkind, lk, ek;
};
__device__ __forceinline__ Decision decide(int ml, int dl, int bl, int me, int de, int be,
                                           int nseg, int &nM, int &nD) {
    const bool zl = ml == kIdZero, il = ml == kIdIdent;
    const bool ze = me == kIdZero, ie = me == kIdIdent;
    const bool dze = de == kIdZero, dzl = dl == kIdZero;
    Decision r;
    r.lk = zl ? kZero : il ? kIdent : kMem;
    r.ek = ze ? kZero : ie ? kIdent : kMem;
    r.mprod = 0;
    r.dkind = 0;
    if ((zl && (ze || !be)) || (ze && !bl)) {
        r.rm = kIdZero;
    } else if (il && !be) {
        r.rm = me;
    } else if (ie && !bl) {
        r.rm = ml;
    } else {
        r.rm = nseg + nM++;
        r.mprod = 1;
    }
    // D part: T = Ml De, then T + Dl
    if ((zl && !be) || (dze && !bl)) {
        r.rd = dl;
    } else if (il && !be) {
        if (dzl) {
            r.rd = de;
        } else {
            r.rd = nseg + nD++;
            r.dkind = 1;
        }
    } else {
        r.rd = nseg + nD++;
        r.dkind = 2;
    }
    return r;
}

// A record of a composition that multiplies: ml, me, rm, lk | ek << 2 | 16
// (M product), dl, de, rd, dkind | dze << 2 | dzl << 3.
__device__ __forceinline__ void put_record(short *pl, int ml, int me, int dl, int de,
                                           const Decision &c) {
    pl[0] = (short)ml; pl[1] = (short)me; pl[2] = (short)c.rm;
    pl[3] = (short)(c.lk | (c.ek << 2) | (c.mprod << 4));
    pl[4] = (short)dl; pl[5] = (short)de; pl[6] = (short)c.rd;
    pl[7] = (short)(c.dkind | ((int)(de == kIdZero) << 2) | ((int)(dl == kIdZero) << 3));
}

// The tree and the outputs, grid (H, P), after blel_flags_kernel.
template <int DK, int DV>
__global__ __launch_bounds__(NTH_TREE, 2) void blel_kernel(int H, int nseg, int size,
                                                           const float *M, const float *D,
                                                           const float *S0, float *S_in,
                                                           float *S_final, BlelWs w, int P,
                                                           uint32_t epoch) {
    const int h = blockIdx.x, wp = blockIdx.y;   // head, workgroup of the head
    // not on the XCD the round-robin dispatch gives the head's first workgroup
    const bool misplaced = P > 1 && xcc_id() != (h & 7);
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    // slot ids (at most nseg + 4 * kMaxSize) and flags
    __shared__ short s_m[kMaxSize + 2], s_d[kMaxSize + 2], s_b[kMaxSize + 2];
    // the compositions that multiply (put_record): one level's, or with the
    // tree in registers every level's, level lv from s_lvl[lv] to s_lvl[lv + 1]
    __shared__ short s_plan[kMaxSize / 2][8];
    __shared__ int s_np;
    __shared__ int s_lvl[2 * 6 + 2];
    constexpr int kPark = kMaxSize + 1;
    const int gw = threadIdx.x / 64, gt = threadIdx.x;
    const int lane = threadIdx.x & 63;
    int rounds = 0;   // barriers passed
    int mixed = 0;    // a workgroup of this head is not on the head's XCD
    // every workgroup of the head has stored what it formed
    auto meet = [&]() __attribute__((always_inline)) {
        if (P > 1) {
            ++rounds;
            head_barrier(w.bar + h, w.bar + H + h, P, rounds, rounds == 1, misplaced, mixed, epoch);
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
    };
    auto mptr = [&](int id) -> const float * {
        return id < 0 ? nullptr : id < nseg ? M + ((int64_t)id * H + h) * mm
                                            : w.Mw + ((int64_t)(id - nseg) * H + h) * mm;
    };
    auto dptr = [&](int id) -> const float * {
        return id < 0 ? nullptr : id < nseg ? D + ((int64_t)id * H + h) * dd
                                            : w.Dw + ((int64_t)(id - nseg) * H + h) * dd;
    };
    // the listed compositions from record k0 to k1, shared out over the head's workgroups
    auto form = [&](int k0, int k1) __attribute__((always_inline)) {
        for (int k = k0 + wp; k < k1; k += P) {
            const short *pl = s_plan[k];
            const int ml = pl[0], me = pl[1], rm = pl[2], mw = pl[3];
            const int dl = pl[4], de = pl[5], rd = pl[6], dw = pl[7];
            if (mw & 16) {
                Acc<DK, DK> am;
                mm_acc<DK, DK>(mptr(ml), mptr(me), am, mw & 3, (mw >> 2) & 3, gw);
                store_acc<DK, DK>(am, nullptr, (float *)mptr(rm), gw);
            }
            if ((dw & 3) == 1) {
                add_n<DK * DV>((float *)dptr(rd), dptr(de), dptr(dl), gt);
            } else if ((dw & 3) == 2) {
                Acc<DK, DV> ad;
                mm_acc<DK, DV>(mptr(ml), dptr(de), ad, mw & 3, (dw & 4) ? kZero : kMem, gw);
                store_acc<DK, DV>(ad, (dw & 8) ? nullptr : dptr(dl), (float *)dptr(rd), gw);
            }
        }
    };
    const bool s0bad = S0 && load_flag(w.s0bad + h);
    // Levels lv < nlev: up-sweep with step 2^lv; lv == nlev: the root takes
    // the identity; lv > nlev: down-sweep with step size / 2^(lv - nlev).
    int nlev = 0;
    while ((1 << nlev) < size) ++nlev;
    int nM = 0, nD = 0;   // fresh buffers used (wave 0's count)
    if (size <= 64) {
        // Wave 0 replays the whole tree with the slots in registers (lane L
        // holds slot L; the spare slot and the root's total are scalars) and
        // lists every composition that multiplies; with none (a zero M
        // everywhere) no workgroup waits for another.
        if (threadIdx.x < 64) {
            int sm, sd, sb;   // this lane's slot
            if (lane < nseg) {
                sm = load_flag(w.fz + lane * H + h) ? lane : kIdZero;
                sd = lane;
                sb = load_flag(w.fb + lane * H + h);
            } else {   // identity padding
                sm = kIdIdent;
                sd = kIdZero;
                sb = 0;
            }
            int tm = 0, td = 0, tb = 0;   // the total (root slot)
            int np = 0;
            auto rd_m = [&](int i) { return __builtin_amdgcn_readlane(sm, i); };
            auto rd_d = [&](int i) { return __builtin_amdgcn_readlane(sd, i); };
            auto rd_b = [&](int i) { return __builtin_amdgcn_readlane(sb, i); };
            for (int lv = 0; lv <= 2 * nlev; ++lv) {
                s_lvl[lv] = np;
                if (lv == nlev) {
                    tm = rd_m(size - 1);
                    td = rd_d(size - 1);
                    tb = rd_b(size - 1);
                    if (lane == size - 1) {
                        sm = kIdIdent;
                        sd = kIdZero;
                        sb = 0;
                    }
                    continue;
                }
                const bool up = lv < nlev;
                const int step = up ? 1 << lv : size >> (lv - nlev);
                for (int i = 2 * step - 1; i < size; i += 2 * step) {
                    int ml, dl, bl;
                    if (up) {
                        ml = rd_m(i); dl = rd_d(i); bl = rd_b(i);
                    } else {
                        // (P[i-step], P[i]) <- (P[i], P[i-step] o P[i])
                        ml = rd_m(i - step); dl = rd_d(i - step); bl = rd_b(i - step);
                        const int pm = rd_m(i), pd = rd_d(i), pb = rd_b(i);
                        if (lane == i - step) {
                            sm = pm;
                            sd = pd;
                            sb = pb;
                        }
                    }
                    const int e = up ? i - step : i;
                    const int me = rd_m(e), de = rd_d(e), be = rd_b(e);
                    const Decision c = decide(ml, dl, bl, me, de, be, nseg, nM, nD);
                    if (c.mprod | c.dkind) put_record(s_plan[np++], ml, me, dl, de, c);
                    if (lane == i) {
                        sm = c.rm;
                        sd = c.rd;
                        sb = bl | be;
                    }
                }
            }
            s_lvl[2 * nlev + 1] = np;
            if (lane < size) {
                s_m[lane] = (short)sm;
                s_d[lane] = (short)sd;
                s_b[lane] = (short)sb;
            }
            if (lane == 0) {
                s_m[size] = (short)tm;
                s_d[size] = (short)td;
                s_b[size] = (short)tb;
            }
        }
        __syncthreads();
        for (int lv = 0; lv <= 2 * nlev; ++lv) {
            const int k0 = s_lvl[lv], k1 = s_lvl[lv + 1];
            if (k1 == k0) continue;
            form(k0, k1);
            meet();   // the products are visible to the next level
        }
    } else {
        // larger trees: slots in LDS; wave 0 replays one level at a time
        for (int j = threadIdx.x; j < size; j += NTH_TREE) {
            if (j < nseg) {
                s_m[j] = (short)(load_flag(w.fz + j * H + h) ? j : kIdZero);
                s_d[j] = (short)j;
                s_b[j] = (short)load_flag(w.fb + j * H + h);
            } else {   // identity padding
                s_m[j] = kIdIdent;
                s_d[j] = kIdZero;
                s_b[j] = 0;
            }
        }
        __syncthreads();
        auto compose = [&](int l, int e, int r, int &np) __attribute__((always_inline)) {
            const int ml = s_m[l], dl = s_d[l], bl = s_b[l];
            const int me = s_m[e], de = s_d[e], be = s_b[e];
            const Decision c = decide(ml, dl, bl, me, de, be, nseg, nM, nD);
            if (c.mprod | c.dkind) put_record(s_plan[np++], ml, me, dl, de, c);
            s_m[r] = (short)c.rm;
            s_d[r] = (short)c.rd;
            s_b[r] = (short)(bl | be);
        };
        for (int lv = 0; lv <= 2 * nlev; ++lv) {
            if (lv == nlev) {
                if (threadIdx.x == 0) {
                    s_m[size] = s_m[size - 1];
                    s_d[size] = s_d[size - 1];
                    s_b[size] = s_b[size - 1];
                    s_m[size - 1] = kIdIdent;
                    s_d[size - 1] = kIdZero;
                    s_b[size - 1] = 0;
                }
                __syncthreads();
                continue;
            }
            const bool up = lv < nlev;
            const int step = up ? 1 << lv : size >> (lv - nlev);
            if (threadIdx.x < 64) {   // a wave's LDS accesses complete in order
                int np = 0;
                for (int i = 2 * step - 1; i < size; i += 2 * step) {
                    int l = i, e = i - step;
                    if (!up) {
                        // (P[i-step], P[i]) <- (P[i], P[i-step] o P[i]); the
                        // old P[i-step] waits in the spare slot
                        s_m[kPark] = s_m[i - step];
                        s_d[kPark] = s_d[i - step];
                        s_b[kPark] = s_b[i - step];
                        s_m[i - step] = s_m[i];
                        s_d[i - step] = s_d[i];
                        s_b[i - step] = s_b[i];
                        l = kPark;
                        e = i;
                    }
                    compose(l, e, i, np);
                }
                s_np = np;
            }
            __syncthreads();
            const int np = s_np;
            form(0, np);
            if (np > 0) meet();      // the products are visible to the next level
            else __syncthreads();    // s_plan and s_np are rewritten by the next level
        }
    }

    // 3. S_in[j] = Pre_j.M S0 + Pre_j.D (slot j), S_final from the total (slot size)
    const float *s0 = S0 ? S0 + (int64_t)h * dd : nullptr;
    for (int j = wp; j <= nseg; j += P) {
        const int slot = j < nseg ? j : size;
        const int idm = s_m[slot], idd = s_d[slot];
        float *out = j < nseg ? S_in + ((int64_t)j * H + h) * dd : S_final + (int64_t)h * dd;
        const float *Ad = dptr(idd);
        if (!s0 || (idm == kIdZero && !s0bad)) {
            copy_n<DK * DV>(out, Ad, gt);   // zeros when Ad is null
        } else if (idm == kIdIdent && !s0bad) {
            if (Ad) add_n<DK * DV>(out, s0, Ad, gt);
            else copy_n<DK * DV>(out, s0, gt);
        } else {
            Acc<DK, DV> acc;
            mm_acc<DK, DV>(mptr(idm), s0, acc, idm == kIdZero ? kZero : idm == kIdIdent ? kIdent : kMem,
                           kMem, gw);
            store_acc<DK, DV>(acc, Ad, out, gw);
        }
    }
}

// ---------------------------------------------------------------------------
// Segments split into f sub-segments (kda_segment_package on a device whose
// compute units the segments alone would leave idle).  Sub-segment k of
// segment j is unit u = f j + k; its packages are computed like a segment's,
// then merged left to right: step k fixes sub-segment k up from the
// accumulated state of sub-segments 0..k-1 (the chunk engine's fix-up mode)
// and composes the packages, P_u <- P_u o P_{u-1}, in place.
// ---------------------------------------------------------------------------

// sb[f j + k] = seg_start[j] + chunk-aligned k/f of segment j, sb[f nseg] = T;
// ord[(k-1) nseg + j] = f j + k for k = 1..f-1.
__global__ void split_bounds_kernel(const int64_t *seg_start, int nseg, int f, int64_t *sb,
                                    int32_t *ord) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx > f * nseg) return;
    if (idx == f * nseg) {
        sb[idx] = seg_start[nseg];
        return;
    }
    const int j = idx / f, k = idx - j * f;
    const int64_t a = seg_start[j], len = seg_start[j + 1] - a;
    sb[idx] = a + (len * k / f) / kChunk * kChunk;
    if (k > 0) ord[(k - 1) * nseg + j] = idx;
}

// Step k of the merge, grid (nseg, H): with u = f j + k,
//   (M_u, D_u) <- (M_u M_{u-1}, M_u D_{u-1} + D_u)
// in place: in the sub-segment slots, or at the last step in M_out[j] and
// D_out[j], where the package launch wrote the last sub-segment's M and D (its
// M stays in slot u when M_out is NULL, and only D is composed).  A zero factor
// is skipped against finite values, and an output that keeps its value is not
// written: with M_u exactly zero (a short memory) the step only reads.
template <int DK, int DV>
__global__ __launch_bounds__(NTH) void split_compose_kernel(int H, int nseg, int f, int k,
                                                            float *Ms, float *Ds, float *M_out,
                                                            float *D_out) {
    const int j = blockIdx.x, h = blockIdx.y;
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    const int64_t u = (int64_t)f * j + k;
    const bool last = k == f - 1;
    float *Ml = last && M_out ? M_out + ((int64_t)j * H + h) * mm : Ms + (u * H + h) * mm;
    float *Dl = last ? D_out + ((int64_t)j * H + h) * dd : Ds + (u * H + h) * dd;
    const float *Me = Ms + ((u - 1) * H + h) * mm, *De = Ds + ((u - 1) * H + h) * dd;
    float *Mo = last && !M_out ? nullptr : Ml;   // M is composed where it is kept
    bool zl, ze, bl, be;
    {
        Tile<DK * DK> tl, te;
        tl.load(Ml);
        te.load(Me);
        zl = !tl.any_nonzero();
        ze = !te.any_nonzero();
        bl = tl.any_nonfinite();
        be = te.any_nonfinite();
    }
    {
        Tile<DK * DV> tl, te;
        tl.load(Dl);
        te.load(De);
        bl = tl.any_nonfinite() || bl;
        be = te.any_nonfinite() || be;
    }
    const bool need_mm = !((zl && ze) || (zl && !be) || (ze && !bl));
    const bool need_md = !(zl && !be);
    Acc<DK, DK> am;
    Acc<DK, DV> ad;
    if (need_mm && Mo) mm_acc<DK, DK>(Ml, Me, am, zl ? kZero : kMem, ze ? kZero : kMem);
    if (need_md) mm_acc<DK, DV>(Ml, De, ad, zl ? kZero : kMem);
    __syncthreads();   // every operand read precedes the first store
    if (Mo) {
        if (need_mm) store_acc<DK, DK>(am, nullptr, Mo);
        else if (!zl) copy_n<DK * DK>(Mo, nullptr);   // a zero M_{u-1} against a finite M_u
    }
    if (need_md) store_acc<DK, DV>(ad, Dl, Dl);
}

// Rungs of the sub-packages inside sub-segment k >= 1 (grid (rows, H)):
// sub_M[r] <- sub_M[r] M_{f j + k - 1}, the map from the segment's start
// instead of the sub-segment's.
template <int DK>
__global__ __launch_bounds__(NTH) void split_rung_m_kernel(int H, int nseg, int f, int k,
                                                           const int64_t *sb, int interval,
                                                           const float *Ms, float *sub_M) {
    const int64_t r = blockIdx.x;
    const int h = blockIdx.y;
    const int64_t p = (r + 1) * interval;
    int u = 0;
    while (u + 1 < f * nseg && sb[u + 1] < p) ++u;   // p in (sb[u], sb[u+1]]
    if (u % f != k) return;
    const int64_t mm = (int64_t)DK * DK;
    float *L = sub_M + (r * H + h) * mm;
    const float *R = Ms + ((int64_t)(u - 1) * H + h) * mm;
    bool zl, zr, bl, br;
    {
        Tile<DK * DK> tl, tr;
        tl.load(L);
        tr.load(R);
        zl = !tl.any_nonzero();
        zr = !tr.any_nonzero();
        bl = tl.any_nonfinite();
        br = tr.any_nonfinite();
    }
    if ((zl && zr) || (zl && !br)) return;   // stays exactly zero
    Acc<DK, DK> am;
    if (!(zr && !bl)) mm_acc<DK, DK>(L, R, am, zl ? kZero : kMem, zr ? kZero : kMem);
    __syncthreads();
    if (zr && !bl) copy_n<DK * DK>(L, nullptr);
    else store_acc<DK, DK>(am, nullptr, L);
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
    mm_acc<DK, DV>(Lm, Sj, acc, nz ? kMem : kZero);
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
                      float *S_in, float *S_final, int *flags, hipStream_t s) {
    if (flags) {
        hipLaunchKernelGGL((seq_flags_kernel<DK>), dim3(nseg, H), dim3(NTH), 0, s, H, M, flags);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((scan_seq_kernel<DK, DV>), dim3(H * (DV / SEQ_CW)), dim3(NTH), 0, s, H,
                       nseg, M, D, S0, S_in, S_final, (const int *)flags);
    return hipGetLastError();
}

template <int DK, int DV>
BlelWs blel_ws(void *ws, int H, int nseg) {
    const int size = pow2_at_least(nseg);
    BlelWs w;
    w.Mw = (float *)ws;
    w.Dw = w.Mw + (int64_t)2 * size * H * DK * DK;
    w.bar = (unsigned long long *)(w.Dw + (int64_t)2 * size * H * DK * DV);
    w.fz = (int *)(w.bar + 2 * (int64_t)H);
    w.fb = w.fz + (int64_t)nseg * H;
    w.s0bad = w.fb + (int64_t)nseg * H;
    return w;
}

// Workgroups per head: up to 8, while H x P is at most half of the
// workgroups the device holds at once (per device, queried once).
template <int DK, int DV>
int blel_width(int H) {
    static std::mutex mu;
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
    int per_dev;
    {
        std::lock_guard<std::mutex> lock(mu);
        per_dev = cached[dev];
    }
    if (per_dev == 0) {
        int cus = 0, nb = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, blel_kernel<DK, DV>, NTH_TREE, 0) !=
            hipSuccess)
            nb = 0;
        per_dev = std::max(1, nb * cus);
        std::lock_guard<std::mutex> lock(mu);
        cached[dev] = per_dev;
    }
    return std::max(1, std::min(8, per_dev / (2 * H)));
}

// A fresh epoch per launch for the barrier counters (odd multiples of a large
// odd constant: never zero, and unlike small integers or common bit patterns).
uint32_t next_epoch() {
    static std::atomic<uint32_t> n{0};
    return (n.fetch_add(1, std::memory_order_relaxed) + 1u) * 0x9E3779B1u | 1u;
}

template <int DK, int DV>
hipError_t scan_blel_t(int H, int nseg, const float *M, const float *D, const float *S0,
                       float *S_in, float *S_final, void *ws, hipStream_t s) {
    const int size = pow2_at_least(nseg);
    if (size > kMaxSize) return hipErrorInvalidValue;
    const BlelWs w = blel_ws<DK, DV>(ws, H, nseg);
    const int P = blel_width<DK, DV>(H);
    hipLaunchKernelGGL((blel_flags_kernel<DK, DV>), dim3(nseg + 1, H), dim3(NTH), 0, s, H, nseg, M,
                       D, S0, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((blel_kernel<DK, DV>), dim3(H, P), dim3(NTH_TREE), 0, s, H, nseg, size, M,
                       D, S0, S_in, S_final, w, P, next_epoch());
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

int blelloch_max_segments() { return kMaxSize; }

size_t blelloch_workspace(int dk, int dv, int H, int nseg) {
    const int size = pow2_at_least(nseg);
    return (size_t)2 * size * H * ((size_t)dk * dk + (size_t)dk * dv) * sizeof(float) +
           (size_t)2 * H * sizeof(unsigned long long) + ((size_t)2 * nseg * H + H) * sizeof(int);
}

size_t sequential_workspace(int H, int nseg) { return (size_t)nseg * H * sizeof(int); }

hipError_t launch_scan_sequential(int dk, int dv, int H, int nseg, const float *M, const float *D,
                                  const float *S0, float *S_in, float *S_final, int *flags,
                                  hipStream_t s) {
    if (dk == 64 && dv == 64) return scan_seq_t<64, 64>(H, nseg, M, D, S0, S_in, S_final, flags, s);
    if (dk == 64 && dv == 128) return scan_seq_t<64, 128>(H, nseg, M, D, S0, S_in, S_final, flags, s);
    if (dk == 128 && dv == 64) return scan_seq_t<128, 64>(H, nseg, M, D, S0, S_in, S_final, flags, s);
    if (dk == 128 && dv == 128) return scan_seq_t<128, 128>(H, nseg, M, D, S0, S_in, S_final, flags, s);
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

hipError_t launch_split_bounds(const int64_t *seg_start, int nseg, int f, int64_t *sb,
                               int32_t *ord, hipStream_t s) {
    const int n = f * nseg + 1;
    hipLaunchKernelGGL(split_bounds_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       seg_start, nseg, f, sb, ord);
    return hipGetLastError();
}

hipError_t launch_split_compose(int dk, int dv, int H, int nseg, int f, int k, float *Ms,
                                float *Ds, float *M_out, float *D_out, hipStream_t s) {
#define KDA_SPLIT_COMPOSE(DK_, DV_)                                                             \
    if (dk == DK_ && dv == DV_) {                                                               \
        hipLaunchKernelGGL((split_compose_kernel<DK_, DV_>), dim3(nseg, H), dim3(NTH), 0, s, H,  \
                           nseg, f, k, Ms, Ds, M_out, D_out);                                   \
        return hipGetLastError();                                                               \
    }
    KDA_SPLIT_COMPOSE(64, 64)
    KDA_SPLIT_COMPOSE(64, 128)
    KDA_SPLIT_COMPOSE(128, 64)
    KDA_SPLIT_COMPOSE(128, 128)
#undef KDA_SPLIT_COMPOSE
    return hipErrorInvalidValue;
}

hipError_t launch_split_rung_m(int dk, int H, int nseg, int f, int k, const int64_t *sb,
                               int interval, int64_t rows, const float *Ms, float *sub_M,
                               hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    if (dk == 64)
        hipLaunchKernelGGL((split_rung_m_kernel<64>), dim3((unsigned)rows, H), dim3(NTH), 0, s, H,
                           nseg, f, k, sb, interval, Ms, sub_M);
    else if (dk == 128)
        hipLaunchKernelGGL((split_rung_m_kernel<128>), dim3((unsigned)rows, H), dim3(NTH), 0, s, H,
                           nseg, f, k, sb, interval, Ms, sub_M);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_plan(const int64_t *cu_seqlens, int32_t n, int32_t *order, hipStream_t s) {
    if (n <= 0 || n > kPlanMax) return hipErrorInvalidValue;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, cu_seqlens, n, order);
    return hipGetLastError();
}

}  // namespace kda
