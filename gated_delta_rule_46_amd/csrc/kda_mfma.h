// kda_mfma.h -- gfx950 MFMA operand policies, global I/O helpers and wave
// primitives shared by the KDA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {
namespace mf {

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
// Hides x's definition from the optimiser (no instruction is emitted): keeps
// each scan step a single DPP add instead of a multiply folded into the first
// step or a step split into a DPP move and an add.
__device__ __forceinline__ float dpp_src(float x) {
    asm("" : "+v"(x));
    return x;
}
// Inclusive prefix sum across the 16 lanes of a DPP row.
__device__ __forceinline__ float scan16(float x) {
    x = dpp_src(x);
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x = dpp_src(x);
    x += row_shr<8>(x);
    return dpp_src(x);
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
    __device__ static void stf(T *p, F8 f) { *(F8 *)p = f; }
    __device__ static void st4(T *p, f32x4 v) { *(F4 *)p = cvt4(v); }
    // the same stores as two 8-byte halves, for rows that are only 8-byte aligned
    __device__ static void stf_h(T *p, F8 f) {
        *(F4 *)p = __builtin_shufflevector(f, f, 0, 1, 2, 3);
        *(F4 *)(p + 4) = __builtin_shufflevector(f, f, 4, 5, 6, 7);
    }
    __device__ static void st8_h(T *p, const float *v) { stf_h(p, cvt8(v)); }
    // sign flip of every element (bit operation, exact)
    __device__ static F8 neg(F8 f) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        return __builtin_bit_cast(F8, __builtin_bit_cast(u32x4, f) ^ 0x80008000u);
    }
    __device__ static F8 cat(F4 a, F4 b) {
        return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    __device__ static void unpack8(F8 f, float *out) {
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 w = __builtin_bit_cast(u32x4, f);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            out[2 * j] = __builtin_bit_cast(float, w[j] << 16);
            out[2 * j + 1] = __builtin_bit_cast(float, w[j] & 0xffff0000u);
        }
    }
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
    __device__ static void unpack8(F8 f, float *out) {
#pragma unroll
        for (int j = 0; j < 4; ++j) { out[j] = f.lo[j]; out[j + 4] = f.hi[j]; }
    }
    __device__ static void st8(T *p, const float *v) {
        *(f32x4 *)p = f32x4{v[0], v[1], v[2], v[3]};
        *(f32x4 *)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
    __device__ static void stf(T *p, F8 f) { *(f32x4 *)p = f.lo; *(f32x4 *)(p + 4) = f.hi; }
    __device__ static void stf_h(T *p, F8 f) { stf(p, f); }
    __device__ static void st8_h(T *p, const float *v) { st8(p, v); }
    __device__ static void st4(T *p, f32x4 v) { *(f32x4 *)p = v; }
    __device__ static F8 neg(F8 f) { return F8{-f.lo, -f.hi}; }
    __device__ static F8 cat(F4 a, F4 b) { return F8{a, b}; }
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


__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace mf
}  // namespace kda
