// Prefix scan over segment pairs (cumulative transition M_i, zero-start state
// S_loc_i): the state entering segment i+1 is M_i S_i + S_loc_i.  Zero-start
// states cannot simply be added for KDA because every token applies a
// token-dependent transition to the incoming state; composing the pairs in
// order recovers each segment's true start state (orkas.ai "Kimi K3
// architecture", section "The cost comes back in the serving stack").
//
// One workgroup per (batch*head, 16-column tile of the state).  The running
// start state tile (dk x 16, fp32) lives in LDS; each step is a dk x dk by
// dk x 16 product in fp32.  starts[0] receives a copy of S0 (or zeros) so the
// pass that follows never reads S0 itself (S0 may alias the final state).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK>
__global__ __launch_bounds__(256) void scan_kernel(ScanArgs a) {
    constexpr int TPR = 256 / DK;            // threads per row
    constexpr int CPT = 16 / TPR;            // columns per thread
    static_assert(TPR * DK == 256 && CPT * TPR == 16, "scan thread map");
    __shared__ float cur[DK][17];
    const int ntile = a.dv / 16;
    const int jt = (int)(blockIdx.x % ntile);
    const int64_t bh = blockIdx.x / ntile;
    const int P = a.n_seg, dv = a.dv;
    const int tid = threadIdx.x, c = tid / TPR, j0 = (tid % TPR) * CPT;
    const int col0 = 16 * jt;

    float x[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        x[j] = a.s0 ? a.s0[bh * DK * dv + (int64_t)c * dv + col0 + j0 + j] : 0.f;
        cur[c][j0 + j] = x[j];
        a.starts[(bh * P) * DK * dv + (int64_t)c * dv + col0 + j0 + j] = x[j];
    }
    for (int i = 0; i + 1 < P; ++i) {
        __syncthreads();
        const float* Mrow = a.m_tr + (bh * P + i) * DK * DK + (int64_t)c * DK;
        const float* Sl = a.s_loc + (bh * P + i) * DK * dv + (int64_t)c * dv + col0 + j0;
#pragma unroll
        for (int j = 0; j < CPT; ++j) x[j] = Sl[j];
        for (int u = 0; u < DK; u += 4) {
            const f32x4 m = *reinterpret_cast<const f32x4*>(Mrow + u);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int j = 0; j < CPT; ++j) x[j] += m[e] * cur[u + e][j0 + j];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            cur[c][j0 + j] = x[j];
            a.starts[(bh * P + i + 1) * DK * dv + (int64_t)c * dv + col0 + j0 + j] = x[j];
        }
    }
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t st) {
    const unsigned nblk = (unsigned)(a.B * a.H * (a.dv / 16));
    switch (a.dk) {
        case 16: hipLaunchKernelGGL(scan_kernel<16>, dim3(nblk), dim3(256), 0, st, a); break;
        case 32: hipLaunchKernelGGL(scan_kernel<32>, dim3(nblk), dim3(256), 0, st, a); break;
        case 64: hipLaunchKernelGGL(scan_kernel<64>, dim3(nblk), dim3(256), 0, st, a); break;
        case 128: hipLaunchKernelGGL(scan_kernel<128>, dim3(nblk), dim3(256), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kda
