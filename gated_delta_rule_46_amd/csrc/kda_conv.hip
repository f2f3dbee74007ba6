// kda_conv.hip -- short causal depthwise convolution over tokens, with a
// per-sequence window state and the segment halo.
//
// KDA's q, k and v pass through a short convolution along the token axis
// before the recurrence (kern PR #44: the varlen stage kernels gather the
// short-conv inputs per sequence and update its window; ROCm/ATOM PR #2709:
// the conv state follows a forked request through a read-side index;
// pegainfer PR #970: a segment publishes its conv halo tail to the next one).
// For channel c of sequence n, with x~ the sequence's inputs preceded by its
// window (the W-1 inputs before its first token):
//
//     y_t[c] = act(bias[c] + sum_{j<W} w[c][j] * x~_{t-W+1+j}[c])
//
// and the new window is the last W-1 rows of x~.  The work is one read and one
// write per element with W multiply-adds: bound by HBM.
//
// conv_kernel: a workgroup of 256 threads covers 128 rows x 256 channels; a
// thread owns 16 rows x 8 consecutive channels (a 16-byte bf16 vector per
// row) and issues all of its loads at once: its 16 rows and the W-1 rows above
// them, which the thread above has just read, so they come from cache and HBM
// sees each input row about once.  32 threads of a wave cover 512 contiguous
// bytes of one row.  Threads whose rows touch a sequence start or end take a
// row-by-row path that reads the window slot where needed.  window_kernel
// stores the new windows in a separate launch, after every read of the old
// ones.

#include "kda_ops.h"

namespace kda {
namespace {

constexpr int kConvThreads = 256;
constexpr int kConvVec = 8;                          // channels per thread
constexpr int kBatch = 16;                           // rows per thread
constexpr int kConvGroups = 32;                      // channel groups per workgroup
constexpr int kConvRows = kBatch * (kConvThreads / kConvGroups);   // 128 rows per workgroup

template <bool BF>
__device__ __forceinline__ void load8(const void *p, int64_t i, float *out) {
    if (BF) {
        const uint4 w = *(const uint4 *)((const uint16_t *)p + i);
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            out[2 * j] = __builtin_bit_cast(float, u[j] << 16);
            out[2 * j + 1] = __builtin_bit_cast(float, u[j] & 0xffff0000u);
        }
    } else {
        const float4 a = *(const float4 *)((const float *)p + i);
        const float4 b = *(const float4 *)((const float *)p + i + 4);
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    }
}

// One row of 8 channels as stored (bf16: 4 words; fp32: 8 words).
template <bool BF> struct RawRow { uint32_t u[BF ? 4 : 8]; };

template <bool BF>
__device__ __forceinline__ void load_raw(const void *p, int64_t i, RawRow<BF> &r) {
    if (BF) {
        const uint4 w = *(const uint4 *)((const uint16_t *)p + i);
        r.u[0] = w.x; r.u[1] = w.y; r.u[2] = w.z; r.u[3] = w.w;
    } else {
        const uint4 a = *(const uint4 *)((const float *)p + i);
        const uint4 b = *(const uint4 *)((const float *)p + i + 4);
        r.u[0] = a.x; r.u[1] = a.y; r.u[2] = a.z; r.u[3] = a.w;
        r.u[4] = b.x; r.u[5] = b.y; r.u[6] = b.z; r.u[7] = b.w;
    }
}

template <bool BF>
__device__ __forceinline__ float raw_at(const RawRow<BF> &r, int j) {
    if (BF) return __builtin_bit_cast(float, (j & 1) ? (r.u[j >> 1] & 0xffff0000u) : (r.u[j >> 1] << 16));
    return bits_f32(r.u[j]);
}

// z * sigmoid(z) with the hardware exp2 and reciprocal (about 1 ulp each)
__device__ __forceinline__ float silu(float z) {
    return z * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-z * 1.4426950408889634f));
}

// 8 bf16 values, converted by the hardware's paired conversion (round to
// nearest even, one instruction per two values; a NaN stays a NaN)
typedef __bf16 conv_bf16x8 __attribute__((ext_vector_type(8)));

template <bool BF>
__device__ __forceinline__ void store8(void *p, int64_t i, const float *v) {
    if (BF) {
        conv_bf16x8 w;
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = (__bf16)v[j];
        *(conv_bf16x8 *)((uint16_t *)p + i) = w;
    } else {
        *(float4 *)((float *)p + i) = make_float4(v[0], v[1], v[2], v[3]);
        *(float4 *)((float *)p + i + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
}

// Raw copy of 8 elements (windows hold inputs bit for bit).
template <bool BF>
__device__ __forceinline__ void copy8(const void *src, int64_t i, void *dst, int64_t o) {
    if (BF) {
        *(uint4 *)((uint16_t *)dst + o) = *(const uint4 *)((const uint16_t *)src + i);
    } else {
        *(float4 *)((float *)dst + o) = *(const float4 *)((const float *)src + i);
        *(float4 *)((float *)dst + o + 4) = *(const float4 *)((const float *)src + i + 4);
    }
}

// Sequence holding row r: the last s with cu[s] <= r (skips empty sequences).
__device__ __forceinline__ int seq_of(const int64_t *cu, int N, int64_t r) {
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= r) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Input at row `row` of the packed tensor as seen by sequence s (rows before
// the sequence's first token come from its window slot, or are zero).
template <bool BF, int W>
__device__ __forceinline__ void input_row(const ConvArgs &a, int s, int64_t row, int c, float *out) {
    const int64_t start = a.cu[s];
    if (row >= start) {
        load8<BF>(a.x, row * a.C + c, out);
        return;
    }
    const int32_t slot = a.read_idx ? a.read_idx[s] : -1;
    const int64_t p = row - start;   // -(W-1) .. -1
    if (slot >= 0 && slot < a.n_slots && p >= -(W - 1)) {
        load8<BF>(a.win, ((int64_t)slot * (W - 1) + (W - 1) + p) * a.C + c, out);
    } else {
#pragma unroll
        for (int j = 0; j < kConvVec; ++j) out[j] = 0.f;
    }
}

// SILU: the activation (a.act == 1), chosen at launch so that neither form
// pays for the other
template <bool BF, int W, bool SILU>
__global__ __launch_bounds__(kConvThreads) void conv_kernel(const ConvArgs a) {
    // thread (rg, cg): rows r0 .. r0+7, channels c .. c+7
    const int cg = threadIdx.x & (kConvGroups - 1), rg = threadIdx.x / kConvGroups;
    const int c = (blockIdx.y * kConvGroups + cg) * kConvVec;
    const int64_t r0 = (int64_t)blockIdx.x * kConvRows + rg * kBatch;
    if (c >= a.C || r0 >= a.T) return;
    const int nr = a.T - r0 < kBatch ? (int)(a.T - r0) : kBatch;
    float w[W][kConvVec], b[kConvVec];
#pragma unroll
    for (int j = 0; j < kConvVec; ++j) {
#pragma unroll
        for (int k = 0; k < W; ++k) w[k][j] = a.weight[(int64_t)(c + j) * W + k];
        b[j] = a.bias ? a.bias[c + j] : 0.f;
    }
    auto out_row = [&](const float (*win)[kConvVec], int64_t r) {
        // win[0 .. W-1]: the W inputs of row r, oldest first
        float y[kConvVec];
#pragma unroll
        for (int j = 0; j < kConvVec; ++j) {
            float acc = b[j];
#pragma unroll
            for (int k = 0; k < W; ++k) acc = fmaf(w[k][j], win[k][j], acc);
            y[j] = SILU ? silu(acc) : acc;
        }
        store8<BF>(a.y, r * a.C + c, y);
    };
    int s = seq_of(a.cu, a.N, r0);
    if (nr == kBatch && r0 - (W - 1) >= a.cu[s] && r0 + kBatch <= a.cu[s + 1]) {
        // all W-1+16 input rows inside one sequence: every load issued at once,
        // kept as stored until used
        RawRow<BF> cat[W - 1 + kBatch];
#pragma unroll
        for (int i = 0; i < W - 1 + kBatch; ++i) load_raw<BF>(a.x, (r0 - (W - 1) + i) * a.C + c, cat[i]);
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            float y[kConvVec];
#pragma unroll
            for (int j = 0; j < kConvVec; ++j) {
                float acc = b[j];
#pragma unroll
                for (int k = 0; k < W; ++k) acc = fmaf(w[k][j], raw_at<BF>(cat[i + k], j), acc);
                y[j] = SILU ? silu(acc) : acc;
            }
            store8<BF>(a.y, (r0 + i) * a.C + c, y);
        }
        return;
    }
    // near a sequence start or end: row by row, each against its own sequence
    for (int i = 0; i < nr; ++i) {
        const int64_t r = r0 + i;
        while (a.cu[s + 1] <= r) ++s;
        float win[W][kConvVec];
#pragma unroll
        for (int k = 0; k < W; ++k) input_row<BF, W>(a, s, r - (W - 1) + k, c, win[k]);
        out_row(win, r);
    }
}

// New window of each sequence: the last W-1 rows of (old window, inputs).
// One thread per (sequence, 8 channels); every value is read before any is
// written, so a slot may be both read and written by its own sequence.
template <bool BF, int W>
__global__ __launch_bounds__(kConvThreads) void window_kernel(const ConvArgs a) {
    const int c = (blockIdx.y * kConvThreads + threadIdx.x) * kConvVec;
    const int s = blockIdx.x;
    if (c >= a.C) return;
    const int32_t ws = a.write_idx[s];
    if (ws < 0 || ws >= a.n_slots) return;
    const int64_t start = a.cu[s], len = a.cu[s + 1] - start;
    float v[W - 1][kConvVec];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) input_row<BF, W>(a, s, start + len - (W - 1) + k, c, v[k]);
#pragma unroll
    for (int k = 0; k < W - 1; ++k) {
        // stored exactly: every value is an input element (or zero)
        const int64_t o = ((int64_t)ws * (W - 1) + k) * a.C + c;
        store8<BF>(a.win, o, v[k]);
    }
}

// Halo tails: the last W-1 input rows before each segment's end (zeros
// before row 0) into slot write_idx[j].
template <bool BF, int W>
__global__ __launch_bounds__(kConvThreads) void halo_kernel(const ConvArgs a) {
    const int c = (blockIdx.y * kConvThreads + threadIdx.x) * kConvVec;
    const int j = blockIdx.x;
    if (c >= a.C) return;
    const int32_t ws = a.write_idx[j];
    if (ws < 0 || ws >= a.n_slots) return;
    const int64_t end = a.cu[j + 1];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) {
        const int64_t row = end - (W - 1) + k;
        const int64_t o = ((int64_t)ws * (W - 1) + k) * a.C + c;
        if (row >= 0) {
            copy8<BF>(a.x, row * a.C + c, a.win, o);
        } else {
            const float z[kConvVec] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            store8<BF>(a.win, o, z);
        }
    }
}

template <bool BF, int W>
hipError_t launch_w(int what, const ConvArgs &a, hipStream_t s) {
    const unsigned cy = (unsigned)((a.C / kConvVec + kConvThreads - 1) / kConvThreads);
    if (what == 0) {
        const int64_t tiles = (a.T + kConvRows - 1) / kConvRows;
        const unsigned cgy = (unsigned)((a.C / kConvVec + kConvGroups - 1) / kConvGroups);
        if (tiles > 0) {
            if (a.act == 1)
                hipLaunchKernelGGL((conv_kernel<BF, W, true>), dim3((unsigned)tiles, cgy),
                                   dim3(kConvThreads), 0, s, a);
            else
                hipLaunchKernelGGL((conv_kernel<BF, W, false>), dim3((unsigned)tiles, cgy),
                                   dim3(kConvThreads), 0, s, a);
        }
        if (a.write_idx && a.N > 0)
            hipLaunchKernelGGL((window_kernel<BF, W>), dim3((unsigned)a.N, cy), dim3(kConvThreads), 0, s, a);
    } else {
        if (a.N > 0)
            hipLaunchKernelGGL((halo_kernel<BF, W>), dim3((unsigned)a.N, cy), dim3(kConvThreads), 0, s, a);
    }
    return hipGetLastError();
}

template <bool BF>
hipError_t launch_bf(int what, int width, const ConvArgs &a, hipStream_t s) {
    switch (width) {
        case 2: return launch_w<BF, 2>(what, a, s);
        case 3: return launch_w<BF, 3>(what, a, s);
        case 4: return launch_w<BF, 4>(what, a, s);
        case 5: return launch_w<BF, 5>(what, a, s);
        case 6: return launch_w<BF, 6>(what, a, s);
        case 7: return launch_w<BF, 7>(what, a, s);
        case 8: return launch_w<BF, 8>(what, a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_conv(bool bf16, int width, const ConvArgs &a, hipStream_t s) {
    return bf16 ? launch_bf<true>(0, width, a, s) : launch_bf<false>(0, width, a, s);
}

hipError_t launch_conv_halo(bool bf16, int width, const ConvArgs &a, hipStream_t s) {
    return bf16 ? launch_bf<true>(1, width, a, s) : launch_bf<false>(1, width, a, s);
}

}  // namespace kda
