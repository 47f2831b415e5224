// Lead form of a segmented prefill plan, for gfx950.
//
// In a segmented plan (orkas.ai "Kimi K3 architecture", section "The cost comes back in the
// serving stack": segments summarised as (cumulative transition, zero-start state) pairs, a
// prefix scan for the true start states, the segments rerun from those) every sequence's
// last segment needs no summary, so pass 1 leaves the compute units of one segment per
// (batch, head) idle.  Segment 0, on the other hand, needs no scan: its start state is S0.
// The lead kernel runs both in one launch: workgroups 0 .. n0-1 run segment 0 of every
// (batch, head, column block) in pass-2 form (from S0, writing o and its final state, the
// true start of segment 1, into the start states), the rest run pass 1 over segments
// 1 .. P-2.  The scan then starts from segment 1 and pass 2 reruns segments 1 .. P-1.
// Segment 0 is shorter than the others (the plan sizes it by the ratio of a pass-1 chunk's
// time to a pass-2 chunk's), so both parts of the launch end together.
#include <mutex>

#include "kda_chunk_body.h"

namespace kda {

// EXT0 / EXT1: the extended instantiation (see chunk_kernel) for segment 0 / for pass 1; pass 1
// has no checkpoints, so a call that asks only for those runs its plain body.
template <typename OpT, int DK, int C, bool EXT0, bool EXT1>
__global__ __launch_bounds__(512) void chunk_lead_kernel(ChunkArgs a0, ChunkArgs a1, int64_t n0) {
    const int64_t bid = blockIdx.x;                // uniform: each workgroup runs one of the two
    if (bid < n0) chunk_body<OpT, DK, C, 0, EXT0>(a0, bid);
    else chunk_body<OpT, DK, C, 1, EXT1>(a1, bid - n0);
}

template <typename OpT, int DK, int C, bool EXT0, bool EXT1>
static hipError_t launch_lead_e(const ChunkArgs& a0, const ChunkArgs& a1, hipStream_t st) {
    constexpr size_t lds = (size_t)lds_layout(sizeof(OpT), DK, C).total;
    auto kern = chunk_lead_kernel<OpT, DK, C, EXT0, EXT1>;
    static std::once_flag once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(once, [&] {
        attr_err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 163840);
    });
    if (attr_err != hipSuccess) return attr_err;
    // segment 0: one workgroup per (batch, head, column block); pass 1: per (batch, head, segment)
    const int64_t n0 = a0.B * a0.H * (int64_t)a0.seg_cnt * (a0.dv / a0.dv_block);
    const int64_t n1 = a1.B * a1.H * (int64_t)a1.seg_cnt;
    if (n0 + n1 <= 0) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3((unsigned)(n0 + n1)), dim3(512), lds, st, a0, a1, n0);
    return hipGetLastError();
}

template <typename OpT, int DK, int C>
static hipError_t launch_lead_c(const ChunkArgs& a0, const ChunkArgs& a1, hipStream_t st) {
    // (float32: chunk * dk <= 4096, as for the chunk kernel)
    if constexpr (sizeof(OpT) == 4 && C * DK > 4096) return hipErrorInvalidValue;
    else {
        if (a0.flags != 0) return launch_lead_e<OpT, DK, C, true, true>(a0, a1, st);
        if (a0.ckpt) return launch_lead_e<OpT, DK, C, true, false>(a0, a1, st);
        return launch_lead_e<OpT, DK, C, false, false>(a0, a1, st);
    }
}

template <typename OpT, int DK>
static hipError_t lead_dispatch_c(const ChunkArgs& a0, const ChunkArgs& a1, hipStream_t st) {
    switch (a0.chunk) {
        case 16: return launch_lead_c<OpT, DK, 16>(a0, a1, st);
        case 32: return launch_lead_c<OpT, DK, 32>(a0, a1, st);
        case 64: return launch_lead_c<OpT, DK, 64>(a0, a1, st);
    }
    return hipErrorInvalidValue;
}

template <typename OpT>
static hipError_t lead_dispatch_dk(const ChunkArgs& a0, const ChunkArgs& a1, hipStream_t st) {
    switch (a0.dk) {
        case 16: return lead_dispatch_c<OpT, 16>(a0, a1, st);
        case 32: return lead_dispatch_c<OpT, 32>(a0, a1, st);
        case 64: return lead_dispatch_c<OpT, 64>(a0, a1, st);
        case 128: return lead_dispatch_c<OpT, 128>(a0, a1, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_lead(const ChunkArgs& a0, const ChunkArgs& a1, hipStream_t st) {
    return a0.bf16 ? lead_dispatch_dk<bf16>(a0, a1, st) : lead_dispatch_dk<float>(a0, a1, st);
}

}  // namespace kda
