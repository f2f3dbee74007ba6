// kda_scan.hip -- (M,D) package scans, segment-path checkpoints and the
// longest-first work plan.
//
// Packages (pegainfer PR #970 "cross-process CP whale gang", whale-lane commit
// text: segments exchange KDA (M,D) packages, combined all-prefix or by a
// Blelloch prefix scan) map a segment's incoming state to S_out = M S_in + D.
// Composition, later after earlier: (Mb,Db) o (Ma,Da) = (Mb Ma, Mb Da + Db).
//
// Every product here is "out[DK x 32] = L[DK x DK] R[DK x 32] + Add" in fp32
// on one workgroup: L staged whole in LDS, the 32-column tile of R in LDS.
// When L is exactly zero (the usual case once a segment has forgotten its
// incoming state) the multiply is skipped and out = Add, which is exact.

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int TC = 32;     // columns per tile
constexpr int NTH = 256;   // threads per workgroup

template <int DK> struct AffineLds {
    static constexpr int LDL = DK + 1;
    static constexpr int LDRT = TC + 1;
    static constexpr int bytes = (DK * LDL + DK * LDRT) * 4 + 64;
};

// Loads L (row-major DK x DK, leading dim DK) into LDS; returns whether any
// element is nonzero (block-uniform).
template <int DK>
__device__ bool stage_left(const float *L, float *sL, int *s_nz) {
    constexpr int LDL = AffineLds<DK>::LDL;
    const int t = threadIdx.x;
    if (t == 0) *s_nz = 0;
    __syncthreads();
    bool nz = false;
    if (L) {
        for (int e = t; e < DK * DK; e += NTH) {
            const float x = L[e];
            sL[(e / DK) * LDL + (e % DK)] = x;
            nz |= (__builtin_bit_cast(uint32_t, x) & 0x7fffffffu) != 0u;
        }
    }
    if (nz) atomicOr(s_nz, 1);
    __syncthreads();
    return *s_nz != 0;
}

// out[:, 0:TC] = sL * R[:, 0:TC] + Add[:, 0:TC]   (R, Add, out row-major with
// their own leading dims; Add may be null; R may alias out only if the caller
// has already staged it -- R is staged into LDS before any store).
template <int DK>
__device__ void affine_tile(const float *sL, bool nz, const float *R, int ldr, const float *Add,
                            int lda, float *out, int ldo, float *sR) {
    constexpr int LDL = AffineLds<DK>::LDL;
    constexpr int LDRT = AffineLds<DK>::LDRT;
    constexpr int TPR = NTH / DK;        // threads per row
    constexpr int CPT = TC / TPR;        // columns per thread
    const int t = threadIdx.x;
    const int r = t / TPR, c0 = (t % TPR) * CPT;
    if (nz) {
        for (int e = t; e < DK * TC; e += NTH) {
            const int rr = e / TC, cc = e % TC;
            sR[rr * LDRT + cc] = R[(int64_t)rr * ldr + cc];
        }
    }
    float acc[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) acc[j] = Add ? Add[(int64_t)r * lda + c0 + j] : 0.f;
    __syncthreads();
    if (nz) {
        for (int k = 0; k < DK; ++k) {
            const float lv = sL[r * LDL + k];
#pragma unroll
            for (int j = 0; j < CPT; ++j) acc[j] = fmaf(lv, sR[k * LDRT + c0 + j], acc[j]);
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < CPT; ++j) out[(int64_t)r * ldo + c0 + j] = acc[j];
}

// ---------------------------------------------------------------------------
// Sequential scan: grid (H, DV/TC).  S_in[0] = S0, S_in[j+1] = M_j S_in[j] + D_j.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(NTH) void scan_seq_kernel(int H, int nseg, const float *M,
                                                       const float *D, const float *S0,
                                                       float *S_in, float *S_final) {
    extern __shared__ __align__(16) unsigned char smem[];
    float *sL = (float *)smem;
    float *sR = sL + DK * AffineLds<DK>::LDL;
    int *s_nz = (int *)(sR + DK * AffineLds<DK>::LDRT);
    const int h = blockIdx.x, col = blockIdx.y * TC;
    const int64_t sstride = (int64_t)DK * DV;
    // S_in[0] = S0 (or zeros)
    for (int e = threadIdx.x; e < DK * TC; e += NTH) {
        const int rr = e / TC, cc = e % TC;
        S_in[(int64_t)h * sstride + rr * DV + col + cc] = S0 ? S0[(int64_t)h * sstride + rr * DV + col + cc] : 0.f;
    }
    __syncthreads();
    for (int j = 0; j < nseg; ++j) {
        const float *Mj = M + ((int64_t)j * H + h) * DK * DK;
        const float *Dj = D + ((int64_t)j * H + h) * sstride + col;
        const float *Sj = S_in + ((int64_t)j * H + h) * sstride + col;
        float *dst = (j + 1 < nseg) ? S_in + ((int64_t)(j + 1) * H + h) * sstride + col
                                    : S_final + (int64_t)h * sstride + col;
        const bool nz = stage_left<DK>(Mj, sL, s_nz);
        affine_tile<DK>(sL, nz, Sj, DV, Dj, DV, dst, DV, sR);
        __threadfence_block();
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Blelloch scan over packages stored in the workspace:
//   Pm [size+1][H][DK][DK], Pd [size+1][H][DK][DV]; slot `size` keeps the total.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ void blel_init_kernel(int H, int nseg, int size, const float *M, const float *D,
                                 float *Pm, float *Pd) {
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    const int64_t totalM = (int64_t)size * H * mm, totalD = (int64_t)size * H * dd;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < totalM + totalD;
         e += (int64_t)gridDim.x * blockDim.x) {
        if (e < totalM) {
            const int64_t slot = e / (H * mm);
            const int64_t within = e % mm;
            Pm[e] = slot < nseg ? M[e] : ((within / DK) == (within % DK) ? 1.f : 0.f);
        } else {
            const int64_t f = e - totalM;
            const int64_t slot = f / (H * dd);
            Pd[f] = slot < nseg ? D[f] : 0.f;
        }
    }
}

// One level: grid (npairs, H).  Pair p touches i = (p+1)*2*step - 1 and
// j = i - step.  Up-sweep: P[i] = P[i] o P[j].  Down-sweep: (P[j], P[i]) =
// (P[i], P[j] o P[i]).  In both, out = Lpkg o Rpkg is written to slot i.
template <int DK, int DV>
__global__ __launch_bounds__(NTH) void blel_level_kernel(int H, int step, int down, float *Pm,
                                                         float *Pd) {
    extern __shared__ __align__(16) unsigned char smem[];
    float *sL = (float *)smem;
    float *sR = sL + DK * AffineLds<DK>::LDL;
    int *s_nz = (int *)(sR + DK * AffineLds<DK>::LDRT);
    const int h = blockIdx.y;
    const int64_t i = (int64_t)(blockIdx.x + 1) * 2 * step - 1, j = i - step;
    const int64_t li = down ? j : i, ri = down ? i : j;
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    float *Lm = Pm + (li * H + h) * mm, *Ld = Pd + (li * H + h) * dd;
    float *Rm = Pm + (ri * H + h) * mm, *Rd = Pd + (ri * H + h) * dd;
    float *Om = Pm + (i * H + h) * mm, *Od = Pd + (i * H + h) * dd;
    float *Jm = Pm + (j * H + h) * mm, *Jd = Pd + (j * H + h) * dd;
    const bool nz = stage_left<DK>(Lm, sL, s_nz);
    // Column tiles of the M part (no addend) and of the D part (addend L.D).
    // Each tile's inputs are read before its outputs are written, tiles are
    // disjoint, and L.M is already in LDS, so the in-place update is safe.
    constexpr int LDRT = AffineLds<DK>::LDRT;
    for (int part = 0; part < 2; ++part) {
        const int ncol = part == 0 ? DK : DV;
        const int ld = ncol;
        float *Rp = part == 0 ? Rm : Rd;
        float *Op = part == 0 ? Om : Od;
        float *Jp = part == 0 ? Jm : Jd;
        const float *Add = part == 0 ? nullptr : Ld;
        for (int col = 0; col < ncol; col += TC) {
            // keep the old R tile (down-sweep copies it to slot j)
            float keep[DK * TC / NTH];
            int kidx = 0;
            for (int e = threadIdx.x; e < DK * TC; e += NTH) {
                const int rr = e / TC, cc = e % TC;
                keep[kidx++] = Rp[(int64_t)rr * ld + col + cc];
            }
            // stage R tile and the addend, compute, then write
            for (int e = threadIdx.x; e < DK * TC; e += NTH) {
                const int rr = e / TC, cc = e % TC;
                sR[rr * LDRT + cc] = Rp[(int64_t)rr * ld + col + cc];
            }
            constexpr int TPR = NTH / DK, CPT = TC / TPR;
            const int r = threadIdx.x / TPR, c0 = (threadIdx.x % TPR) * CPT;
            float acc[CPT];
#pragma unroll
            for (int q = 0; q < CPT; ++q) acc[q] = Add ? Add[(int64_t)r * ld + col + c0 + q] : 0.f;
            __syncthreads();
            if (nz) {
                for (int k = 0; k < DK; ++k) {
                    const float lv = sL[r * AffineLds<DK>::LDL + k];
#pragma unroll
                    for (int q = 0; q < CPT; ++q) acc[q] = fmaf(lv, sR[k * LDRT + c0 + q], acc[q]);
                }
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < CPT; ++q) Op[(int64_t)r * ld + col + c0 + q] = acc[q];
            if (down) {
                kidx = 0;
                for (int e = threadIdx.x; e < DK * TC; e += NTH) {
                    const int rr = e / TC, cc = e % TC;
                    Jp[(int64_t)rr * ld + col + cc] = keep[kidx++];
                }
            }
            __syncthreads();
        }
    }
}

// After the up-sweep: slot `size` = total, slot size-1 = identity.
template <int DK, int DV>
__global__ void blel_root_kernel(int H, int size, float *Pm, float *Pd) {
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < H * (mm + dd);
         e += (int64_t)gridDim.x * blockDim.x) {
        if (e < H * mm) {
            float *src = Pm + (int64_t)(size - 1) * H * mm + e;
            Pm[(int64_t)size * H * mm + e] = *src;
            const int64_t within = e % mm;
            *src = (within / DK) == (within % DK) ? 1.f : 0.f;
        } else {
            const int64_t f = e - H * mm;
            float *src = Pd + (int64_t)(size - 1) * H * dd + f;
            Pd[(int64_t)size * H * dd + f] = *src;
            *src = 0.f;
        }
    }
}

// S_in[j] = P[j].M S0 + P[j].D (j < nseg);  S_final = P[size].M S0 + P[size].D.
// grid (nseg+1, H, DV/TC).
template <int DK, int DV>
__global__ __launch_bounds__(NTH) void blel_apply_kernel(int H, int nseg, int size, const float *Pm,
                                                         const float *Pd, const float *S0,
                                                         float *S_in, float *S_final) {
    extern __shared__ __align__(16) unsigned char smem[];
    float *sL = (float *)smem;
    float *sR = sL + DK * AffineLds<DK>::LDL;
    int *s_nz = (int *)(sR + DK * AffineLds<DK>::LDRT);
    const int jj = blockIdx.x, h = blockIdx.y, col = blockIdx.z * TC;
    const int slot = jj < nseg ? jj : size;
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    const float *Lm = Pm + ((int64_t)slot * H + h) * mm;
    const float *Ad = Pd + ((int64_t)slot * H + h) * dd + col;
    float *out = (jj < nseg ? S_in + ((int64_t)jj * H + h) * dd : S_final + (int64_t)h * dd) + col;
    const bool nz = S0 ? stage_left<DK>(Lm, sL, s_nz) : false;
    affine_tile<DK>(sL, nz, S0 ? S0 + (int64_t)h * dd + col : nullptr, DV, Ad, DV, out, DV, sR);
}

// Segment-path checkpoints: grid (rows, H, DV/TC).  Rung row r sits at
// p = (r+1)*interval inside segment j (seg_start[j] < p <= seg_start[j+1]).
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
    const int h = blockIdx.y, col = blockIdx.z * TC;
    const int64_t p = (r + 1) * interval;
    int j = 0;
    while (j + 1 < nseg && seg_start[j + 1] < p) ++j;
    const int64_t mm = (int64_t)DK * DK, dd = (int64_t)DK * DV;
    const bool nz = stage_left<DK>(sub_M + (r * H + h) * mm, sL, s_nz);
    affine_tile<DK>(sL, nz, S_in + ((int64_t)j * H + h) * dd + col, DV,
                    sub_D + (r * H + h) * dd + col, DV, states + (r * H + h) * dd + col, DV, sR);
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

template <int DK, int DV>
hipError_t scan_seq_t(int H, int nseg, const float *M, const float *D, const float *S0,
                      float *S_in, float *S_final, hipStream_t s) {
    const int lds = AffineLds<DK>::bytes;
    hipError_t e = set_lds(scan_seq_kernel<DK, DV>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((scan_seq_kernel<DK, DV>), dim3(H, DV / TC), dim3(NTH), lds, s, H, nseg,
                       M, D, S0, S_in, S_final);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t scan_blel_t(int H, int nseg, const float *M, const float *D, const float *S0,
                       float *S_in, float *S_final, void *ws, hipStream_t s) {
    int size = 1;
    while (size < nseg) size *= 2;
    float *Pm = (float *)ws;
    float *Pd = Pm + (int64_t)(size + 1) * H * DK * DK;
    const int lds = AffineLds<DK>::bytes;
    hipError_t e;
    hipLaunchKernelGGL((blel_init_kernel<DK, DV>), dim3(1024), dim3(256), 0, s, H, nseg, size, M,
                       D, Pm, Pd);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = set_lds(blel_level_kernel<DK, DV>, lds)) != hipSuccess) return e;
    for (int step = 1; step < size; step *= 2) {
        hipLaunchKernelGGL((blel_level_kernel<DK, DV>), dim3(size / (2 * step), H), dim3(NTH), lds,
                           s, H, step, 0, Pm, Pd);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL((blel_root_kernel<DK, DV>), dim3(256), dim3(256), 0, s, H, size, Pm, Pd);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    for (int step = size / 2; step >= 1; step /= 2) {
        hipLaunchKernelGGL((blel_level_kernel<DK, DV>), dim3(size / (2 * step), H), dim3(NTH), lds,
                           s, H, step, 1, Pm, Pd);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = set_lds(blel_apply_kernel<DK, DV>, lds)) != hipSuccess) return e;
    hipLaunchKernelGGL((blel_apply_kernel<DK, DV>), dim3(nseg + 1, H, DV / TC), dim3(NTH), lds, s,
                       H, nseg, size, Pm, Pd, S0, S_in, S_final);
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
    hipLaunchKernelGGL((ckpt_kernel<DK, DV>), dim3((unsigned)rows, H, DV / TC), dim3(NTH), lds, s, H,
                       nseg, seg_start, interval, S_in, sub_M, sub_D, states);
    return hipGetLastError();
}

}  // namespace

size_t blelloch_workspace(int dk, int dv, int H, int nseg) {
    int size = 1;
    while (size < nseg) size *= 2;
    return (size_t)(size + 1) * H * ((size_t)dk * dk + (size_t)dk * dv) * sizeof(float);
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
