// kda_decode.hip -- one-token KDA step per sequence against a pool of states.
//
// Decode is the recurrence with a single token (KDA: S <- Diag(alpha) S, then
// S <- S + beta k (v - S^T k)^T, o = S^T q).  The state of each sequence lives
// in a caller-owned pool and is addressed by two slot indices, one read and
// one written, so a forked request resumes a shared prefix state without a
// copy (ROCm/ATOM PR #2709: the fused sigmoid-gated delta-rule update takes a
// read-side state index beside the write table).  The gates can arrive as
// logits: beta = sigmoid(b) and log alpha = -softplus(a), evaluated in-kernel.
//
// The work is a pass over the state (64 KiB of fp32 per head at d = 128) with
// two reductions over the key dimension, so the kernel is bound by HBM.  One
// workgroup of four waves handles one (sequence, head, 64-column block): lane
// (cq, ro) of wave w owns columns 4cq..4cq+3 and rows 16j + 4w + ro, held in
// registers from the read to the write.  A wave reads four 256-byte row
// segments per instruction.

#include "kda_ops.h"

namespace kda {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecCols = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool BF>
__device__ __forceinline__ float ld1(const void *p, int64_t i) {
    if (BF) return __builtin_bit_cast(float, (uint32_t)((const uint16_t *)p)[i] << 16);
    return ((const float *)p)[i];
}

template <bool BF>
__device__ __forceinline__ f32x4 ld4(const void *p, int64_t i) {
    if (BF) {
        const uint2 w = *(const uint2 *)((const uint16_t *)p + i);
        return f32x4{__builtin_bit_cast(float, w.x << 16), __builtin_bit_cast(float, w.x & 0xffff0000u),
                     __builtin_bit_cast(float, w.y << 16), __builtin_bit_cast(float, w.y & 0xffff0000u)};
    }
    return *(const f32x4 *)((const float *)p + i);
}

// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <bool BF>
__device__ __forceinline__ void st4(void *p, int64_t i, f32x4 v) {
    if (BF) {
        uint2 w;
        w.x = bf16_bits(v[0]) | (bf16_bits(v[1]) << 16);
        w.y = bf16_bits(v[2]) | (bf16_bits(v[3]) << 16);
        *(uint2 *)((uint16_t *)p + i) = w;
    } else {
        *(f32x4 *)((float *)p + i) = v;
    }
}

// Sum of x over the four lane groups that share a column quad (lanes cq,
// cq+16, cq+32, cq+48).
__device__ __forceinline__ f32x4 reduce_groups(f32x4 x) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        x[c] += __shfl_xor(x[c], 16);
        x[c] += __shfl_xor(x[c], 32);
    }
    return x;
}

template <int DK, int DV, bool BF>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(const DecodeArgs a) {
    constexpr int NCB = DV / kDecCols;
    constexpr int NS = DK / 16;   // row steps per lane
    __shared__ float s_q[DK], s_k[DK], s_a[DK];
    __shared__ __align__(16) float s_r[4][kDecCols];
    __shared__ __align__(16) float s_o[4][kDecCols];
    __shared__ float s_norm[4][2];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int cq = lane & 15, ro = lane >> 4;
    const int H = a.H;
    const int cb = blockIdx.x % NCB;
    const int item = blockIdx.x / NCB;   // grid covers N*H items exactly
    const int n = item / H, h = item - n * H;
    const int col = cb * kDecCols + 4 * cq;
    const int64_t ss = (int64_t)DK * DV;
    const int rs = a.read_idx[n], wsl = a.write_idx[n];
    const bool rd = rs >= 0 && rs < a.n_slots;
    const bool wr = wsl >= 0 && wsl < a.n_slots;

    // state rows first: the longest latency of the step
    f32x4 S[NS];
    if (rd) {
        const float *src = a.pool + ((int64_t)rs * H + h) * ss + col;
#pragma unroll
        for (int j = 0; j < NS; ++j) S[j] = *(const f32x4 *)(src + (int64_t)(16 * j + 4 * w + ro) * DV);
    } else {
#pragma unroll
        for (int j = 0; j < NS; ++j) S[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // token inputs, norms and gates (thread t < DK owns key channel t)
    const int64_t tk = (int64_t)n * H + h;
    float qv = 0.f, kv = 0.f, gv = 0.f;
    if (tid < DK) {
        qv = ld1<BF>(a.q, tk * DK + tid);
        kv = ld1<BF>(a.k, tk * DK + tid);
        gv = a.g[tk * DK + tid];
    }
    float sq = qv * qv, sk = kv * kv;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        sq += __shfl_xor(sq, off);
        sk += __shfl_xor(sk, off);
    }
    if (lane == 0) { s_norm[w][0] = sq; s_norm[w][1] = sk; }
    __syncthreads();
    const float tq = s_norm[0][0] + s_norm[1][0] + s_norm[2][0] + s_norm[3][0];
    const float tkk = s_norm[0][1] + s_norm[1][1] + s_norm[2][1] + s_norm[3][1];
    const float fq = a.l2norm ? a.scale * rsqrtf(tq + 1e-6f) : a.scale;
    const float fk = a.l2norm ? rsqrtf(tkk + 1e-6f) : 1.f;
    float bt = a.beta[tk];
    if (a.gate_logits) {
        // log alpha = -softplus(a) = -(max(a,0) + log1p(exp(-|a|))); beta = sigmoid(b)
        gv = -(fmaxf(gv, 0.f) + log1pf(expf(-fabsf(gv))));
        bt = 1.f / (1.f + expf(-bt));
    }
    if (tid < DK) {
        s_q[tid] = qv * fq;
        s_k[tid] = kv * fk;
        s_a[tid] = expf(gv);
    }
    __syncthreads();

    // decay, then r = S^T k
    f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int row = 16 * j + 4 * w + ro;
        S[j] *= s_a[row];
        r += s_k[row] * S[j];
    }
    r = reduce_groups(r);
    if (ro == 0) *(f32x4 *)&s_r[w][4 * cq] = r;
    __syncthreads();
    const f32x4 rt = *(const f32x4 *)&s_r[0][4 * cq] + *(const f32x4 *)&s_r[1][4 * cq] +
                     *(const f32x4 *)&s_r[2][4 * cq] + *(const f32x4 *)&s_r[3][4 * cq];
    const f32x4 u = bt * (ld4<BF>(a.v, tk * DV + col) - rt);

    // write along k, read out with q, store the new state
    f32x4 oacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        const int row = 16 * j + 4 * w + ro;
        S[j] += s_k[row] * u;
        oacc += s_q[row] * S[j];
    }
    if (wr) {
        float *dst = a.pool + ((int64_t)wsl * H + h) * ss + col;
#pragma unroll
        for (int j = 0; j < NS; ++j) *(f32x4 *)(dst + (int64_t)(16 * j + 4 * w + ro) * DV) = S[j];
    }
    oacc = reduce_groups(oacc);
    if (ro == 0) *(f32x4 *)&s_o[w][4 * cq] = oacc;
    __syncthreads();
    if (w == 0 && ro == 0) {
        const f32x4 ov = *(const f32x4 *)&s_o[0][4 * cq] + *(const f32x4 *)&s_o[1][4 * cq] +
                         *(const f32x4 *)&s_o[2][4 * cq] + *(const f32x4 *)&s_o[3][4 * cq];
        st4<BF>(a.o, tk * DV + col, ov);
    }
}

template <int DK, int DV, bool BF>
hipError_t launch_dec(const DecodeArgs &a, hipStream_t s) {
    const int64_t grid = (int64_t)a.N * a.H * (DV / kDecCols);
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((decode_kernel<DK, DV, BF>), dim3((unsigned)grid), dim3(kDecThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

bool decode_supported(int dk, int dv) {
    return (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
}

hipError_t launch_decode(bool bf16, int dk, int dv, const DecodeArgs &a, hipStream_t s) {
    if (!decode_supported(dk, dv)) return hipErrorInvalidValue;
#define KDA_DEC(DK_, DV_)                                                            \
    if (dk == DK_ && dv == DV_)                                                      \
        return bf16 ? launch_dec<DK_, DV_, true>(a, s) : launch_dec<DK_, DV_, false>(a, s);
    KDA_DEC(64, 64)
    KDA_DEC(64, 128)
    KDA_DEC(128, 64)
    KDA_DEC(128, 128)
#undef KDA_DEC
    return hipErrorInvalidValue;
}

}  // namespace kda
