// Device-side helpers shared by the KDA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int WAVE = 64;
constexpr float LOG2E = 1.4426950408889634f;
// Floor of the log-decay: every step keeps at least e^-5 ~ 0.67 % of the state
// (orkas.ai "Kimi K3 architecture", section "The floor that removed a GPU code
// path").  The upper clamp at 0 keeps every decay factor <= 1.
constexpr float LOG_ALPHA_FLOOR = -5.0f;

// One v_med3_f32 (fminf / fmaxf would first quiet signalling NaNs with an extra v_max_f32 per
// value); a NaN input gives the floor, as fmaxf(NaN, -5) does.
__device__ __forceinline__ float clamp_log_alpha(float x) {
    return __builtin_amdgcn_fmed3f(x, LOG_ALPHA_FLOOR, 0.0f);
}

// e^x through the hardware 2^x unit.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * LOG2E); }
// 2^x (hardware v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Log-decay from a raw gate logit x through an activation that stops at the floor:
// -5 sigmoid(x) = -5 / (1 + e^-x), in (-5, 0).  The floor constant is what made the
// gate's activation need a lower bound (orkas.ai "Kimi K3 architecture", section "The
// floor that removed a GPU code path"); the sigmoid form is this library's reading.
// Large logits decay fastest; e^-x overflowing to inf gives 0 (no decay).
__device__ __forceinline__ float gate_from_logit(float x) {
    return clamp_log_alpha(LOG_ALPHA_FLOOR * __builtin_amdgcn_rcpf(1.0f + fast_exp(-x)));
}
// Gate input -> floored log-decay; gate 0: the input is the log-decay, 1: a raw logit.
__device__ __forceinline__ float log_decay(float x, int gate) {
    return gate ? gate_from_logit(x) : clamp_log_alpha(x);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

}  // namespace kda
