// Chunked KDA prefill for gfx950: the chunk kernel (one pass, segment pass 1, segment pass 2)
// and its launchers.  The work of one workgroup, and the method it follows, is in
// kda_chunk_body.h.
#include <mutex>

#include "kda_chunk_body.h"

namespace kda {

// ---------------------------------------------------------------- the kernel
// MODE 0: outputs and final states; MODE 1: segment summaries (see ChunkArgs).
// EXT: the optional features of a call (state checkpoints in MODE 0, gate logits, q / k
// normalisation), switched by the arguments at run time.  A separate instantiation: their
// code, even never taken, costs the plain loop several per cent.
template <typename OpT, int DK, int C, int MODE, bool EXT>
__global__ __launch_bounds__(512) void chunk_kernel(ChunkArgs a) {
    chunk_body<OpT, DK, C, MODE, EXT>(a, blockIdx.x);
}

// ---------------------------------------------------------------- launch
template <typename OpT, int DK, int C, int MODE, bool EXT>
static hipError_t launch_chunk_m(const ChunkArgs& a, hipStream_t st) {
    constexpr size_t lds = (size_t)lds_layout(sizeof(OpT), DK, C).total;
    auto kern = chunk_kernel<OpT, DK, C, MODE, EXT>;
    // once per instantiation (the attribute belongs to the function, not to a device); calls
    // from several host threads wait for the first
    static std::once_flag once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(once, [&] {
        attr_err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, 163840);
    });
    if (attr_err != hipSuccess) return attr_err;
    // MODE 1: one workgroup per (batch, head, segment) holds every column of [S | M]
    const int nblk_col = MODE == 0 ? a.dv / a.dv_block : 1;
    const int64_t nblk = a.B * a.H * (int64_t)a.seg_cnt * nblk_col;
    if (nblk <= 0) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(512), lds, st, a);
    return hipGetLastError();
}

template <typename OpT, int DK, int C>
static hipError_t launch_chunk_t(const ChunkArgs& a, hipStream_t st) {
    // float32 operands need chunk * dk <= 4096 (LDS); the ABI rejects larger ones before any
    // launch, so they are not instantiated
    if constexpr (sizeof(OpT) == 4 && C * DK > 4096) return hipErrorInvalidValue;
    else {
        const bool ext = a.flags != 0 || (a.mode == 0 && a.ckpt);
        if (a.mode == 1)
            return ext ? launch_chunk_m<OpT, DK, C, 1, true>(a, st) : launch_chunk_m<OpT, DK, C, 1, false>(a, st);
        return ext ? launch_chunk_m<OpT, DK, C, 0, true>(a, st) : launch_chunk_m<OpT, DK, C, 0, false>(a, st);
    }
}

template <typename OpT, int DK>
static hipError_t dispatch_c(const ChunkArgs& a, hipStream_t st) {
    switch (a.chunk) {
        case 16: return launch_chunk_t<OpT, DK, 16>(a, st);
        case 32: return launch_chunk_t<OpT, DK, 32>(a, st);
        case 64: return launch_chunk_t<OpT, DK, 64>(a, st);
    }
    return hipErrorInvalidValue;
}

template <typename OpT>
static hipError_t dispatch_dk(const ChunkArgs& a, hipStream_t st) {
    switch (a.dk) {
        case 16: return dispatch_c<OpT, 16>(a, st);
        case 32: return dispatch_c<OpT, 32>(a, st);
        case 64: return dispatch_c<OpT, 64>(a, st);
        case 128: return dispatch_c<OpT, 128>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_chunk(const ChunkArgs& a, hipStream_t st) {
    return a.bf16 ? dispatch_dk<bf16>(a, st) : dispatch_dk<float>(a, st);
}

}  // namespace kda
