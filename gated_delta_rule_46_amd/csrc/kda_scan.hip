// kda_scan.hip -- (M,D) package scans, segment-path checkpoints and the
// longest-first work plan.
//
// Packages (pegainfer PR #970 "cross-process CP whale gang", whale-lane commit
// text: segments exchange KDA (M,D) packages, combined all-prefix or by a
// Blelloch prefix scan) map a segment's incoming state to S_out = M S_in + D.
// Composition, later after earlier: (Mb,Db) o (Ma,Da) = (Mb Ma, Mb Da + Db).
//
// Every product here is "out[DK x cols] = L[DK x DK] R[DK x cols] + Add" in
// fp32 on one workgroup: L is staged whole in LDS (and tested for being all
// zeros on the way in), R 32 columns at a time.  A zero L -- the usual case
// once a segment has forgotten its incoming state -- turns the product into a
// copy of Add, which is exact.  Copies use 16-byte accesses.

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int TC = 32;     // columns per GEMM tile
constexpr int NTH = 256;   // threads per workgroup

template <int DK> struct AffineLds {
    static constexpr int LDL = DK + 4;     // keeps 16-byte alignment of rows
    static constexpr int LDRT = TC + 1;
    static constexpr int bytes = (DK * LDL + DK * LDRT) * 4 + 64;
};

__device__ __forceinline__ bool nonzero4(float4 x) {
    const uint32_t m = 0x7fffffffu;
    return ((__builtin_bit_cast(uint32_t, x.x) & m) | (__builtin_bit_cast(uint32_t, x.y) & m) |
            (__builtin_bit_cast(uint32_t, x.z) & m) | (__builtin_bit_cast(uint32_t, x.w) & m)) != 0u;
}

// Stages L (row-major DK x DK) into LDS; returns whether any element is nonzero
// (block-uniform).
template <int DK>
__device__ bool stage_left(const float *L, float *sL, int *s_nz) {
    constexpr int LDL = AffineLds<DK>::LDL;
    const int t = threadIdx.x;
    if (t == 0) *s_nz = 0;
    __syncthreads();
    bool nz = false;
    for (int e = t; e < DK * DK / 4; e += NTH) {
        const float4 x = ((const float4 *)L)[e];
        const int r = (e * 4) / DK, c = (e * 4) % DK;
        *(float4 *)(sL + r * LDL + c) = x;
        nz |= nonzero4(x);
    }
    if (nz) atomicOr(s_nz, 1);
    __syncthreads();
    const bool res = *s_nz != 0;
    __syncthreads();
    return res;
}

// Block-uniform test of a DK x DK matrix for a nonzero element.
template <int DK>
__device__ bool any_nonzero(const float *L, int *s_nz) {
    const int t = threadIdx.x;
    if (t == 0) *s_nz = 0;
    __syncthreads();
    bool nz = false;
    for (int e = t; e < DK * DK / 4; e += NTH) nz |= nonzero4(((const float4 *)L)[e]);
    if (nz) atomicOr(s_nz, 1);
    __syncthreads();
    const bool res = *s_nz != 0;
    __syncthreads();
    return res;
}

// out[:, 0:TC] = sL * R[:, 0:TC] + Add[:, 0:TC].  R is staged in LDS before any
// store, so out may alias R; Add may alias out (each element is read by the
// thread that writes it, before it writes).  Add may be null.
template <int DK>
__device__ void gemm_tile(const float *sL, const float *R, int ldr, const float *Add, int lda,
                          float *out, int ldo, float *sR) {
    constexpr int LDL = AffineLds<DK>::LDL;
    constexpr int LDRT = AffineLds<DK>::LDRT;
    constexpr int TPR = NTH / DK;        // threads per row
    constexpr int CPT = TC / TPR;        // columns per thread
    const int t = threadIdx.x;
    const int r = t / TPR, c0 = (t % TPR) * CPT;
    for (int e = t; e < DK * TC; e += NTH) {
        const int rr = e / TC, cc = e % TC;
        sR[rr * LDRT + cc] = R[(int64_t)rr * ldr + cc];
    }
    float acc[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) acc[j] = Add ? Add[(int64_t)r * lda + c0 + j] : 0.f;
    __syncthreads();
    for (int k = 0; k < DK; ++k) {
        const float lv = sL[r * LDL + k];
#pragma unroll
        for (int j = 0; j < CPT; ++j) acc[j] = fmaf(lv, sR[k * LDRT + c0 + j], acc[j]);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < CPT; ++j) out[(int64_t)r * ldo + c0 + j] = acc[j];
}

// dst = src for a contiguous block of n floats (n % 4 == 0), or zeros if src is null.
__device__ __forceinline__ void copy_block(float *dst, const float *src, int64_t n) {
    for (int64_t e = threadIdx.x; e < n / 4; e += NTH)
        ((float4 *)dst)[e] = src ? ((const float4 *)src)[e] : make_float4(0.f, 0.f, 0.f, 0.f);
}

// out = L * R + Add over all `ncol` columns (row-major DK x ncol), L in sL.
template <int DK>
__device__ void affine_full(const float *sL, bool nz, const float *R, const float *Add, float *out,
                            int ncol, float *sR) {
    if (!nz) {
        copy_block(out, Add, (int64_t)DK * ncol);
        return;
    }
    for (int col = 0; col < ncol; col += TC)
        gemm_tile<DK>(sL, R + col, ncol, Add ? Add + col : nullptr, ncol, out + col, ncol, sR);
}

// ---------------------------------------------------------------------------
// Sequential scan: one workgroup per head.  S_in[0] = S0, S_in[j+1] = M_j S_in[j] + D_j.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(NTH) void scan_seq_kernel(int H, int nseg, const float *M,
                                                       const float *D, const float *S0,
                                                       float *S_in, float *S_final) {
    extern __shared__ __align__(16) unsigned char smem[];
    float *sL = (float *)smem;
    float *sR = sL + DK * AffineLds<DK>::LDL;
    int *s_nz = (int *)(sR + DK * AffineLds<DK>::LDRT);
    const int h = blockIdx.x;
    const int64_t ss = (int64_t)DK * DV;
    copy_block(S_in + (int64_t)h * ss, S0 ? S0 + (int64_t)h * ss : nullptr, ss);
    __syncthreads();
    for (int j = 0; j < nseg; ++j) {
        const float *Sj = S_in + ((int64_t)j * H + h) * ss;
        float *dst = (j + 1 < nseg) ? S_in + ((int64_t)(j + 1) * H + h) * ss : S_final + (int64_t)h * ss;
        const bool nz = stage_left<DK>(M + ((int64_t)j * H + h) * DK * DK, sL, s_nz);
        affine_full<DK>(sL, nz, Sj, D + ((int64_t)j * H + h) * ss, dst, DV, sR);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Blelloch scan over packages in the workspace:
//   Pm [size+1][H][DK][DK], Pd [size+1][H][DK][DV], Fz [size+1][H] (1 = M may
//   be nonzero); slot `size` keeps the total.  One workgroup per (pair, head),
//   so each pair's slots are touched by one workgroup only.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(NTH) void blel_init_kernel(int H, int nseg, const float *M,
                                                        const float *D, float *Pm, float *Pd,
                                                        int *Fz) {
    __shared__ int s_nz;
    const int slot = blockIdx.x, h = blockIdx.y;
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    float *pm = Pm + ((int64_t)slot * H + h) * mm;
    float *pd = Pd + ((int64_t)slot * H + h) * dd;
    if (slot < nseg) {
        const float *m = M + ((int64_t)slot * H + h) * mm;
        copy_block(pm, m, mm);
        copy_block(pd, D + ((int64_t)slot * H + h) * dd, dd);
        const bool nz = any_nonzero<DK>(m, &s_nz);
        if (threadIdx.x == 0) Fz[slot * H + h] = nz ? 1 : 0;
    } else {
        for (int e = threadIdx.x; e < mm; e += NTH) pm[e] = (e / DK == e % DK) ? 1.f : 0.f;
        copy_block(pd, nullptr, dd);
        if (threadIdx.x == 0) Fz[slot * H + h] = 1;
    }
}

template <int DK, int DV>
__global__ __launch_bounds__(NTH) void blel_level_kernel(int H, int step, int down, float *Pm,
                                                         float *Pd, int *Fz) {
    extern __shared__ __align__(16) unsigned char smem[];
    float *sL = (float *)smem;
    float *sR = sL + DK * AffineLds<DK>::LDL;
    int *s_nz = (int *)(sR + DK * AffineLds<DK>::LDRT);
    const int h = blockIdx.y;
    const int64_t i = (int64_t)(blockIdx.x + 1) * 2 * step - 1, j = i - step;
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    float *Mi = Pm + (i * H + h) * mm, *Di = Pd + (i * H + h) * dd;
    float *Mj = Pm + (j * H + h) * mm, *Dj = Pd + (j * H + h) * dd;
    const int fi = Fz[i * H + h], fj = Fz[j * H + h];
    if (!down) {
        // P[i] = P[i] o P[j] = (Mi Mj, Mi Dj + Di); unchanged when Mi == 0
        if (!fi) return;
        const bool nz = stage_left<DK>(Mi, sL, s_nz);
        if (nz) {
            for (int col = 0; col < DK; col += TC) gemm_tile<DK>(sL, Mj + col, DK, nullptr, 0, Mi + col, DK, sR);
            for (int col = 0; col < DV; col += TC) gemm_tile<DK>(sL, Dj + col, DV, Di + col, DV, Di + col, DV, sR);
        }
        if (threadIdx.x == 0) Fz[i * H + h] = (nz && fj) ? 1 : 0;
        return;
    }
    // down-sweep: (P[j], P[i]) = (P[i], P[j] o P[i]) with P[j] o P[i] = (Mj Mi, Mj Di + Dj)
    const bool nz = fj ? stage_left<DK>(Mj, sL, s_nz) : false;
    if (!nz) {
        // Mj == 0: P[j] <- P[i]; P[i] <- (0, Dj), element by element
        for (int64_t e = threadIdx.x; e < mm / 4; e += NTH) {
            ((float4 *)Mj)[e] = ((const float4 *)Mi)[e];
            ((float4 *)Mi)[e] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        for (int64_t e = threadIdx.x; e < dd / 4; e += NTH) {
            const float4 a = ((const float4 *)Di)[e], b = ((const float4 *)Dj)[e];
            ((float4 *)Dj)[e] = a;
            ((float4 *)Di)[e] = b;
        }
        if (threadIdx.x == 0) { Fz[j * H + h] = fi; Fz[i * H + h] = 0; }
        return;
    }
    // general case, column tile by column tile: the tile of P[i] is staged
    // before it is overwritten, Mj is in LDS
    for (int part = 0; part < 2; ++part) {
        const int ncol = part == 0 ? DK : DV;
        float *Rp = part == 0 ? Mi : Di;
        float *Jp = part == 0 ? Mj : Dj;
        for (int col = 0; col < ncol; col += TC) {
            // old P[i] tile -> registers (for P[j]) and the product into P[i]
            float keep[DK * TC / NTH];
            int kq = 0;
            for (int e = threadIdx.x; e < DK * TC; e += NTH) keep[kq++] = Rp[(int64_t)(e / TC) * ncol + col + e % TC];
            float addv[DK * TC / NTH];
            kq = 0;
            if (part == 1)
                for (int e = threadIdx.x; e < DK * TC; e += NTH) addv[kq++] = Dj[(int64_t)(e / TC) * ncol + col + e % TC];
            __syncthreads();
            gemm_tile<DK>(sL, Rp + col, ncol, nullptr, 0, Rp + col, ncol, sR);
            __syncthreads();   // the product tile was written with a different thread mapping
            // add Dj (old) to the D part, then move the old P[i] tile to P[j]
            kq = 0;
            for (int e = threadIdx.x; e < DK * TC; e += NTH) {
                const int64_t idx = (int64_t)(e / TC) * ncol + col + e % TC;
                if (part == 1) Rp[idx] += addv[kq];
                Jp[idx] = keep[kq];
                ++kq;
            }
            __syncthreads();
        }
    }
    if (threadIdx.x == 0) { Fz[j * H + h] = fi; Fz[i * H + h] = fi ? 1 : 0; }
}

// After the up-sweep: slot `size` = total, slot size-1 = identity.
template <int DK, int DV>
__global__ __launch_bounds__(NTH) void blel_root_kernel(int H, int size, float *Pm, float *Pd,
                                                        int *Fz) {
    const int h = blockIdx.x;
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    float *lm = Pm + ((int64_t)(size - 1) * H + h) * mm, *ld = Pd + ((int64_t)(size - 1) * H + h) * dd;
    float *tm = Pm + ((int64_t)size * H + h) * mm, *td = Pd + ((int64_t)size * H + h) * dd;
    for (int64_t e = threadIdx.x; e < mm / 4; e += NTH) {
        const float4 x = ((const float4 *)lm)[e];
        ((float4 *)tm)[e] = x;
        const int r = (int)((4 * e) / DK), c = (int)((4 * e) % DK);
        ((float4 *)lm)[e] = make_float4(r == c ? 1.f : 0.f, r == c + 1 ? 1.f : 0.f,
                                        r == c + 2 ? 1.f : 0.f, r == c + 3 ? 1.f : 0.f);
    }
    for (int64_t e = threadIdx.x; e < dd / 4; e += NTH) {
        ((float4 *)td)[e] = ((const float4 *)ld)[e];
        ((float4 *)ld)[e] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (threadIdx.x == 0) { Fz[size * H + h] = Fz[(size - 1) * H + h]; Fz[(size - 1) * H + h] = 1; }
}

// S_in[j] = P[j].M S0 + P[j].D (j < nseg);  S_final = P[size].M S0 + P[size].D.
// grid (nseg+1, H).
template <int DK, int DV>
__global__ __launch_bounds__(NTH) void blel_apply_kernel(int H, int nseg, int size, const float *Pm,
                                                         const float *Pd, const int *Fz,
                                                         const float *S0, float *S_in, float *S_final) {
    extern __shared__ __align__(16) unsigned char smem[];
    float *sL = (float *)smem;
    float *sR = sL + DK * AffineLds<DK>::LDL;
    int *s_nz = (int *)(sR + DK * AffineLds<DK>::LDRT);
    const int jj = blockIdx.x, h = blockIdx.y;
    const int slot = jj < nseg ? jj : size;
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    const float *Lm = Pm + ((int64_t)slot * H + h) * mm;
    const float *Ad = Pd + ((int64_t)slot * H + h) * dd;
    float *out = jj < nseg ? S_in + ((int64_t)jj * H + h) * dd : S_final + (int64_t)h * dd;
    const bool nz = (S0 && Fz[slot * H + h]) ? stage_left<DK>(Lm, sL, s_nz) : false;
    affine_full<DK>(sL, nz, S0 ? S0 + (int64_t)h * dd : nullptr, Ad, out, DV, sR);
}

// Segment-path checkpoints: grid (rows, H).  Rung row r sits at
// p = (r+1)*interval inside segment j (seg_start[j] < p <= seg_start[j+1]):
// states[r] = sub_M[r] S_in[j] + sub_D[r].
template <int DK, int DV>
__global__ __launch_bounds__(NTH) void ckpt_kernel(int H, int nseg, const int64_t *seg_start,
                                                   int interval, const float *S_in,
                                                   const float *sub_M, const float *sub_D,
                                                   float *states) {
    extern __shared__ __align__(16) unsigned char smem[];
    float *sL = (float *)smem;
    float *sR = sL + DK * AffineLds<DK>::LDL;
    int *s_nz = (int *)(sR + DK * AffineLds<DK>::LDRT);
    const int64_t r = blockIdx.x;
    const int h = blockIdx.y;
    const int64_t p = (r + 1) * interval;
    int j = 0;
    while (j + 1 < nseg && seg_start[j + 1] < p) ++j;
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    const bool nz = stage_left<DK>(sub_M + (r * H + h) * mm, sL, s_nz);
    affine_full<DK>(sL, nz, S_in + ((int64_t)j * H + h) * dd, sub_D + (r * H + h) * dd,
                    states + (r * H + h) * dd, DV, sR);
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

template <typename K>
hipError_t set_lds(K kern, int bytes) {
    return hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

int pow2_at_least(int n) {
    int size = 1;
    while (size < n) size *= 2;
    return size;
}

template <int DK, int DV>
hipError_t scan_seq_t(int H, int nseg, const float *M, const float *D, const float *S0,
                      float *S_in, float *S_final, hipStream_t s) {
    const int lds = AffineLds<DK>::bytes;
    hipError_t e = set_lds(scan_seq_kernel<DK, DV>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((scan_seq_kernel<DK, DV>), dim3(H), dim3(NTH), lds, s, H, nseg, M, D, S0,
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
    const int lds = AffineLds<DK>::bytes;
    hipError_t e;
    hipLaunchKernelGGL((blel_init_kernel<DK, DV>), dim3(size, H), dim3(NTH), 0, s, H, nseg, M, D, Pm,
                       Pd, Fz);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = set_lds(blel_level_kernel<DK, DV>, lds)) != hipSuccess) return e;
    for (int step = 1; step < size; step *= 2) {
        hipLaunchKernelGGL((blel_level_kernel<DK, DV>), dim3(size / (2 * step), H), dim3(NTH), lds,
                           s, H, step, 0, Pm, Pd, Fz);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL((blel_root_kernel<DK, DV>), dim3(H), dim3(NTH), 0, s, H, size, Pm, Pd, Fz);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    for (int step = size / 2; step >= 1; step /= 2) {
        hipLaunchKernelGGL((blel_level_kernel<DK, DV>), dim3(size / (2 * step), H), dim3(NTH), lds,
                           s, H, step, 1, Pm, Pd, Fz);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = set_lds(blel_apply_kernel<DK, DV>, lds)) != hipSuccess) return e;
    hipLaunchKernelGGL((blel_apply_kernel<DK, DV>), dim3(nseg + 1, H), dim3(NTH), lds, s, H, nseg,
                       size, Pm, Pd, Fz, S0, S_in, S_final);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t ckpt_t(int H, int64_t T, const int64_t *seg_start, int nseg, int interval,
                  const float *S_in, const float *sub_M, const float *sub_D, float *states,
                  hipStream_t s) {
    const int64_t rows = T / interval;
    if (rows == 0) return hipSuccess;
    const int lds = AffineLds<DK>::bytes;
    hipError_t e = set_lds(ckpt_kernel<DK, DV>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((ckpt_kernel<DK, DV>), dim3((unsigned)rows, H), dim3(NTH), lds, s, H, nseg,
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
    if (dk == 128 && dv == 128) return scan_seq_t<128, 128>(H, nseg, M, D, S0, S_in, S_final, s);
    return hipErrorInvalidValue;
}

hipError_t launch_scan_blelloch(int dk, int dv, int H, int nseg, const float *M, const float *D,
                                const float *S0, float *S_in, float *S_final, void *ws,
                                hipStream_t s) {
    if (dk == 64 && dv == 64) return scan_blel_t<64, 64>(H, nseg, M, D, S0, S_in, S_final, ws, s);
    if (dk == 128 && dv == 128) return scan_blel_t<128, 128>(H, nseg, M, D, S0, S_in, S_final, ws, s);
    return hipErrorInvalidValue;
}

hipError_t launch_ckpt_write(int dk, int dv, int H, int64_t T, const int64_t *seg_start, int nseg,
                             int interval, const float *S_in, const float *sub_M,
                             const float *sub_D, float *states, hipStream_t s) {
    if (dk == 64 && dv == 64)
        return ckpt_t<64, 64>(H, T, seg_start, nseg, interval, S_in, sub_M, sub_D, states, s);
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
