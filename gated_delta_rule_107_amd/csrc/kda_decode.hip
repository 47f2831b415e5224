// Recurrent decode step: one token per sequence, state updated in place.
//
// Per (sequence n, head h), with D = Diag(exp(g)) and g the floored log-decay:
//     DS = D S;  p = (DS)^T k;  r = (DS)^T q;  u = beta (v - p)
//     S <- DS + k u^T;  o = r + (k . q) u        ( = S_new^T q )
// The state is O(1) per sequence and the step cost does not grow with the
// context (llm-wiki.hwlabs.dev, "Kimi K3 ... linear attention", section
// "1. Limits of softmax attention and KDA's direction"); it is updated in place
// (orkas.ai "Kimi K3 architecture", section "The cost comes back in the
// serving stack").
//
// HBM-bound: the fp32 state is read once and written once; everything else is
// a few hundred bytes per (n, h).  One workgroup per (n, h); thread (rg, cg)
// holds rows rg, rg+RG, ... of the 4 state columns cg*4..cg*4+3 in registers,
// so the state never leaves registers between its load and its store.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <typename ET, int DK, int DV>
__global__ __launch_bounds__(256) void decode_kernel(
    float* __restrict__ state, const ET* __restrict__ q, const ET* __restrict__ k,
    const ET* __restrict__ v, const float* __restrict__ log_alpha,
    const float* __restrict__ beta, ET* __restrict__ o) {
    constexpr int CG = DV / 4;                               // float4 column groups
    constexpr int RG = (DK < 256 / CG) ? DK : 256 / CG;      // row groups
    constexpr int RPT = DK / RG;                             // rows per thread
    constexpr int NT = CG * RG;
    constexpr int NWV = NT / WAVE;
    static_assert(NT % WAVE == 0 && NT <= 256 && DK <= NT, "decode thread map");

    const size_t unit = blockIdx.x;
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;

    __shared__ float s_a[DK], s_k[DK], s_q[DK];
    __shared__ f32x4 s_p[NWV][CG], s_r[NWV][CG];
    __shared__ float s_kq[NWV];

    f32x4* S = reinterpret_cast<f32x4*>(state + unit * (size_t)(DK * DV));
    f32x4 sv[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) sv[i] = __builtin_nontemporal_load(&S[(rg + i * RG) * CG + cg]);

    float kq = 0.f;
    if (tid < DK) {
        const float a = fast_exp(clamp_log_alpha(log_alpha[unit * DK + tid]));
        const float kk = to_f32(k[unit * DK + tid]);
        const float qq = to_f32(q[unit * DK + tid]);
        s_a[tid] = a;
        s_k[tid] = kk;
        s_q[tid] = qq;
        kq = kk * qq;
    }
#pragma unroll
    for (int m = WAVE / 2; m >= 1; m >>= 1) kq += __shfl_xor(kq, m);
    if ((tid & (WAVE - 1)) == 0) s_kq[tid / WAVE] = kq;
    __syncthreads();

    f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + i * RG;
        sv[i] *= s_a[row];
        p += sv[i] * s_k[row];
        r += sv[i] * s_q[row];
    }
    // reduce over the row groups that share a wave (lanes differing in bits >= log2 CG)
#pragma unroll
    for (int m = CG; m < WAVE; m <<= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            p[j] += __shfl_xor(p[j], m);
            r[j] += __shfl_xor(r[j], m);
        }
    }
    if ((tid & (WAVE - 1)) < CG) {
        s_p[tid / WAVE][cg] = p;
        s_r[tid / WAVE][cg] = r;
    }
    __syncthreads();

    f32x4 P = s_p[0][cg], R = s_r[0][cg];
    float KQ = s_kq[0];
#pragma unroll
    for (int w = 1; w < NWV; ++w) {
        P += s_p[w][cg];
        R += s_r[w][cg];
        KQ += s_kq[w];
    }
    const float b = beta[unit];
    f32x4 u;
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = b * (to_f32(v[unit * DV + cg * 4 + j]) - P[j]);

#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int row = rg + i * RG;
        __builtin_nontemporal_store(sv[i] + s_k[row] * u, &S[row * CG + cg]);
    }
    if (rg == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) o[unit * DV + cg * 4 + j] = from_f32<ET>(R[j] + KQ * u[j]);
    }
}

template <typename ET, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
    constexpr int CG = DV / 4;
    constexpr int RG = (DK < 256 / CG) ? DK : 256 / CG;
    const unsigned nblk = (unsigned)(a.N * a.H);
    hipLaunchKernelGGL((decode_kernel<ET, DK, DV>), dim3(nblk), dim3(CG * RG), 0, st,
                       a.state, (const ET*)a.q, (const ET*)a.k, (const ET*)a.v, a.log_alpha,
                       a.beta, (ET*)a.o);
    return hipGetLastError();
}

template <typename ET, int DK>
static hipError_t dispatch_dv(const DecodeArgs& a, hipStream_t st) {
    switch (a.dv) {
        case 16: return launch_decode_t<ET, DK, 16>(a, st);
        case 32: return launch_decode_t<ET, DK, 32>(a, st);
        case 64: return launch_decode_t<ET, DK, 64>(a, st);
        case 128: return launch_decode_t<ET, DK, 128>(a, st);
    }
    return hipErrorInvalidValue;
}

template <typename ET>
static hipError_t dispatch_dk(const DecodeArgs& a, hipStream_t st) {
    switch (a.dk) {
        case 16: return dispatch_dv<ET, 16>(a, st);
        case 32: return dispatch_dv<ET, 32>(a, st);
        case 64: return dispatch_dv<ET, 64>(a, st);
        case 128: return dispatch_dv<ET, 128>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
    return a.bf16 ? dispatch_dk<bf16>(a, st) : dispatch_dk<float>(a, st);
}

}  // namespace kda
