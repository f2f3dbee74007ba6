// kda_validate.hip -- debug check of the device-side inputs.
//
// The calls validate their arguments on the host, not the data behind the
// device pointers: that would need a host synchronisation per call.  These
// kernels count, on the device, the input values outside what the kernels
// assume, into int32 counters the caller reads when it wants to (a debug
// run): unit bounds out of order (cu_seqlens, or segment starts off the chunk
// grid; kern PR #44, "k3: flash-kda builds a varlen variant", and pegainfer PR
// #970, whale-lane commit, give the two index forms), log-decays g above zero
// (a decay alpha = e^g above one) or not finite, 16-token blocks whose summed
// g leaves the range the chunk engine's exponentials stay in, and betas that
// are not finite.
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kValThreads = 256;
constexpr int kBlock16 = 16;           // the engine's row block (its reference points)
constexpr float kBlockFloor = -80.f;   // lowest summed log-decay of a row block

// report[0..fields) = 0 (a kernel, not a memset: callers may capture the call)
__global__ void report_clear_kernel(int *report, int fields) {
    if ((int)threadIdx.x < fields) report[threadIdx.x] = 0;
}

// bounds[0] == 0, bounds[n] == T, non-decreasing; with `aligned`, every
// interior bound a multiple of the chunk.  One count per entry at fault.
__global__ void bounds_check_kernel(const int64_t *b, int n, int64_t T, int aligned, int *report) {
    int bad = 0;
    for (int i = threadIdx.x; i <= n; i += blockDim.x) {
        const int64_t x = b[i];
        const bool wrong = (i == 0 && x != 0) || (i == n && x != T) || (i > 0 && x < b[i - 1]) ||
                           (aligned && i > 0 && i < n && x % kChunk != 0);
        bad += wrong ? 1 : 0;
    }
    if (bad) atomicAdd(&report[0], bad);
}

// One thread per (token, four channels of one head).  g > 0 and non-finite g
// are counted per element; a thread whose token starts a 16-token block of its
// unit (blocks counted from the unit's first token) sums the block's g over
// its four channels and counts each channel below kBlockFloor; the thread on a
// head's first four channels also checks that token's beta.
__global__ __launch_bounds__(kValThreads) void g_check_kernel(const float *g, const float *beta,
                                                              const int64_t *b, int n, int64_t T,
                                                              int H, int dk, int *report) {
    const int64_t per = (int64_t)H * dk / 4;   // quads per token
    const int64_t q = (int64_t)blockIdx.x * kValThreads + threadIdx.x;
    if (q >= T * per) return;
    const int64_t t = q / per;
    const int64_t e = (q - t * per) * 4;       // element within the token's row of H * dk
    const int64_t row = (int64_t)H * dk;
    int pos = 0, nonfin = 0, low = 0, bnf = 0;
    if (g) {
        const float4 x = *(const float4 *)(g + t * row + e);
        const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pos += xv[c] > 0.f ? 1 : 0;
            nonfin += __builtin_isfinite(xv[c]) ? 0 : 1;
        }
        int64_t s0 = 0, s1 = T;   // the unit holding t
        if (b) {
            int lo = 0, hi = n - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (b[mid] <= t) lo = mid; else hi = mid - 1;
            }
            s0 = b[lo];
            s1 = b[lo + 1];
        }
        if (t >= s0 && (t - s0) % kBlock16 == 0) {
            float sum[4] = {0.f, 0.f, 0.f, 0.f};
            // (bounds at fault can point past T: the rows read stay below T)
            for (int j = 0; j < kBlock16 && t + j < s1 && t + j < T; ++j) {
                const float4 y = *(const float4 *)(g + (t + j) * row + e);
                sum[0] += y.x; sum[1] += y.y; sum[2] += y.z; sum[3] += y.w;
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) low += sum[c] < kBlockFloor ? 1 : 0;
        }
    }
    if (beta && e % dk == 0) bnf = __builtin_isfinite(beta[t * H + e / dk]) ? 0 : 1;
    if (pos) atomicAdd(&report[1], pos);
    if (nonfin) atomicAdd(&report[2], nonfin);
    if (low) atomicAdd(&report[3], low);
    if (bnf) atomicAdd(&report[4], bnf);
}

}  // namespace

hipError_t launch_validate(int64_t T, int H, int dk, const int64_t *bounds, int n, int aligned,
                           const float *g, const float *beta, int *report, int fields,
                           hipStream_t s) {
    hipLaunchKernelGGL(report_clear_kernel, dim3(1), dim3(64), 0, s, report, fields);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (bounds) {
        hipLaunchKernelGGL(bounds_check_kernel, dim3(1), dim3(kValThreads), 0, s, bounds, n, T,
                           aligned, report);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int64_t threads = T * H * dk / 4;
    if ((g || beta) && threads > 0) {
        const int64_t blocks = (threads + kValThreads - 1) / kValThreads;
        if (blocks > INT32_MAX) return hipErrorInvalidValue;
        hipLaunchKernelGGL(g_check_kernel, dim3((unsigned)blocks), dim3(kValThreads), 0, s, g, beta,
                           bounds, n, T, H, dk, report);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace kda
