// Prefix scan over segment pairs (cumulative transition M_i, zero-start state
// S_loc_i): the state entering segment i+1 is M_i S_i + S_loc_i.  Zero-start
// states cannot simply be added for KDA because every token applies a
// token-dependent transition to the incoming state; composing the pairs in
// order recovers each segment's true start state (orkas.ai "Kimi K3
// architecture", section "The cost comes back in the serving stack").
//
// One workgroup per (batch*head, 16-column tile of the state); wave w owns
// state rows 16w..16w+15.  Each step is a dk x dk by dk x 16
// product per tile on v_mfma_f32_16x16x32_bf16 with both operands split into
// bf16 high and low parts (hi*hi + hi*lo + lo*hi, fp32 accumulation: about 16
// mantissa bits), started from S_loc_i in the accumulator.  The running start
// state sits in LDS transposed (column-major), so each lane reads its 8
// contraction values with two 16-byte loads; the next segment's transition rows
// are loaded into registers while the current step runs.  One extra wave copies
// each start state from LDS to HBM: the product waves issue only loads, so their
// in-order memory counter never makes a step wait for the previous step's stores.
// starts[0] receives a copy of S0 (or zeros), so the pass that follows never
// reads S0 itself (S0 may alias the final state).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

namespace {

__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        hi[j] = (bf16)x[j];
        lo[j] = (bf16)(x[j] - (float)hi[j]);
    }
}

}  // namespace

// CT: 16-column tiles per workgroup
template <int DK, int CT>
__global__ __launch_bounds__(576) void scan_kernel(ScanArgs a) {
    constexpr int NW = DK / 16;                   // waves: one 16-row tile of the state each
    constexpr int KSTEP = (DK + 31) / 32;         // 32-deep MFMA steps over the contraction
    constexpr int LDT = 32 * KSTEP + 4;           // transposed row length (zero padded)
    __shared__ __attribute__((aligned(16))) float curT[16 * CT * LDT];

    // The column blocks of one (batch, head) are 8 block indices apart, so they run on one
    // XCD (workgroups go round-robin over the 8 XCDs) and share its L2 copy of M_i.
    const int nblk = a.dv / (16 * CT);
    int64_t bh;
    int jb;
    {
        const int64_t bid = blockIdx.x, nbh = a.B * a.H;
        const int64_t grp = bid / (8 * nblk), rem = bid % (8 * nblk);
        bh = grp * 8 + rem % 8;
        jb = (int)(rem / 8);
        const int64_t tail0 = (nbh / 8) * 8;
        if (grp * 8 >= tail0) {
            const int64_t ntail = nbh - tail0, r2 = bid - tail0 * nblk;
            bh = tail0 + r2 % ntail;
            jb = (int)(r2 / ntail);
        }
    }
    const int P = a.n_seg, dv = a.dv;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int m = lane & 15, g = lane >> 4;
    const int col0 = 16 * CT * jb + m;            // column of this lane in tile 0 (B / C layouts)
    const int row0 = 16 * w;

    const bool storer = w == NW;                  // the extra wave: LDS -> HBM copies only

    for (int i = threadIdx.x; i < 16 * CT * LDT; i += 64 * (NW + 1)) curT[i] = 0.f;
    __syncthreads();

    // the store wave writes start state i (in curT) to starts[i]; rows are spread over lanes
    auto store_start = [&](int i) {
        float* dst = a.starts + (bh * P + i) * DK * dv + 16 * CT * jb;
        for (int e = lane; e < DK * CT * 4; e += 64) {            // (row, column quad)
            const int row = e / (CT * 4), cq = e % (CT * 4);
            f32x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = curT[(4 * cq + j) * LDT + row];
            *reinterpret_cast<f32x4*>(dst + (int64_t)row * dv + 4 * cq) = v;
        }
    };

    // start state: rows row0 + 4g + r of each tile's column
    if (!storer) {
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            f32x4 cur;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t idx = (int64_t)(row0 + 4 * g + r) * dv + col0 + 16 * c;
                cur[r] = a.s0 ? a.s0[bh * DK * dv + idx] : 0.f;
            }
            *reinterpret_cast<f32x4*>(curT + (16 * c + m) * LDT + row0 + 4 * g) = cur;
        }
    }

    // transition rows of step i: lane (m, g) holds M_i[row0 + m][32 s + 8 g + j]
    float mrow[KSTEP][8];
    f32x4 sl[CT];
    auto load_step = [&](int i) {
        const float* M = a.m_tr + (bh * P + i) * DK * DK + (int64_t)(row0 + m) * DK;
#pragma unroll
        for (int s = 0; s < KSTEP; ++s) {
            const int k0 = 32 * s + 8 * g;
            if (k0 < DK) {
                const f32x4 lo4 = *reinterpret_cast<const f32x4*>(M + k0);
                const f32x4 hi4 = *reinterpret_cast<const f32x4*>(M + k0 + 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    mrow[s][j] = lo4[j];
                    mrow[s][4 + j] = hi4[j];
                }
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) mrow[s][j] = 0.f;
            }
        }
        const float* L = a.s_loc + (bh * P + i) * DK * dv;
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) sl[c][r] = L[(int64_t)(row0 + 4 * g + r) * dv + col0 + 16 * c];
    };
    if (P > 1 && !storer) load_step(0);

    for (int i = 0; i + 1 < P; ++i) {
        __syncthreads();                          // curT holds the start of segment i
        if (storer) {
            store_start(i);
            __syncthreads();
            continue;
        }
        bf16x8 ahi[KSTEP], alo[KSTEP];
#pragma unroll
        for (int s = 0; s < KSTEP; ++s) split8(mrow[s], ahi[s], alo[s]);
        f32x4 acc[CT], acc2[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) {
            acc[c] = sl[c];
            acc2[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        if (i + 2 < P) load_step(i + 1);          // next transition loads during this step
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
            for (int s = 0; s < KSTEP; ++s) {
                const float* src = curT + (16 * c + m) * LDT + 32 * s + 8 * g;
                const f32x4 b0 = *reinterpret_cast<const f32x4*>(src);
                const f32x4 b1 = *reinterpret_cast<const f32x4*>(src + 4);
                float x[8];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[j] = b0[j];
                    x[4 + j] = b1[j];
                }
                bf16x8 bhi, blo;
                split8(x, bhi, blo);
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[s], bhi, acc[c], 0, 0, 0);
                acc2[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[s], blo, acc2[c], 0, 0, 0);
                acc2[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[s], bhi, acc2[c], 0, 0, 0);
            }
        __syncthreads();                          // every wave has read curT
#pragma unroll
        for (int c = 0; c < CT; ++c)
            *reinterpret_cast<f32x4*>(curT + (16 * c + m) * LDT + row0 + 4 * g) = acc[c] + acc2[c];
    }
    __syncthreads();
    if (storer) store_start(P - 1);
}

template <int DK>
static hipError_t launch_scan_dk(const ScanArgs& a, hipStream_t st) {
    const int ct = 1;
    const unsigned nblk = (unsigned)(a.B * a.H * (a.dv / (16 * ct)));
    const dim3 block(64 * (DK / 16 + 1));
    switch (ct) {
        case 1: hipLaunchKernelGGL((scan_kernel<DK, 1>), dim3(nblk), block, 0, st, a); break;
        case 2: hipLaunchKernelGGL((scan_kernel<DK, 2>), dim3(nblk), block, 0, st, a); break;
        case 4: hipLaunchKernelGGL((scan_kernel<DK, 4>), dim3(nblk), block, 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t st) {
    switch (a.dk) {
        case 16: return launch_scan_dk<16>(a, st);
        case 32: return launch_scan_dk<32>(a, st);
        case 64: return launch_scan_dk<64>(a, st);
        case 128: return launch_scan_dk<128>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
