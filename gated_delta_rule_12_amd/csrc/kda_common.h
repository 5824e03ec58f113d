// Device-side helpers and launch declarations shared by the KDA kernels.
// gfx950 (CDNA4) only: 64-wide wavefronts, MFMA matrix cores, 160 KiB LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

// ---------------------------------------------------------------------------
// Scalar conversions.  bf16 is carried as its 16 raw bits.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Activation element type: fp32 or bf16 (raw bits).
template <bool BF16> struct Act;
template <> struct Act<false> {
    using T = float;
    __device__ static __forceinline__ float load(const T* p, size_t i) { return p[i]; }
};
template <> struct Act<true> {
    using T = uint16_t;
    __device__ static __forceinline__ float load(const T* p, size_t i) { return bf16_to_f32(p[i]); }
};

template <bool BF16> __device__ __forceinline__ void store_out(void* o, size_t i, float x);
template <> __device__ __forceinline__ void store_out<false>(void* o, size_t i, float x) {
    static_cast<float*>(o)[i] = x;
}
template <> __device__ __forceinline__ void store_out<true>(void* o, size_t i, float x) {
    // gfx950 converts with round-to-nearest-even in one instruction
    static_cast<uint16_t*>(o)[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// ---------------------------------------------------------------------------
// Forget-gate forms (kda_gate): log2 of alpha from the value as given.
// softplus(x) / ln 2 = max(x, 0) log2(e) + log2(1 + 2^(-|x| log2(e))).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float log2_alpha_from_softplus_arg(float x) {
    constexpr float kLog2e = 1.4426950408889634f;
    const float t = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
    return -(fmaxf(x, 0.f) * kLog2e + __builtin_amdgcn_logf(1.f + t));
}

// alpha = 1 / (1 + e^x) itself (the same gate, for the kernels that multiply
// decay factors instead of adding logarithms); 0 and 1 at the extremes, never
// above 1.
__device__ __forceinline__ float alpha_from_softplus_arg(float x) {
    constexpr float kLog2e = 1.4426950408889634f;
    const float t = __builtin_amdgcn_exp2f(-fabsf(x) * kLog2e);
    return (x > 0.f ? t : 1.f) * __builtin_amdgcn_rcpf(1.f + t);
}

// ---------------------------------------------------------------------------
// Host-side launchers (defined next to their kernels).
// ---------------------------------------------------------------------------
hipError_t launch_recurrent_step(const void* q, const void* k, const void* v,
                                 const void* gate, int gate_kind, const float* beta, float* state,
                                 void* o, int N, int H, int Dk, int Dv,
                                 bool act_bf16, bool out_bf16, hipStream_t stream);

}  // namespace kda
