// Prefix scan over segment pairs (cumulative transition M_i, zero-start state
// S_loc_i): the state entering segment i+1 is M_i S_i + S_loc_i.  Zero-start
// states cannot simply be added for KDA because every token applies a
// token-dependent transition to the incoming state; composing the pairs in
// order recovers each segment's true start state (orkas.ai "Kimi K3
// architecture", section "The cost comes back in the serving stack").
//
// One workgroup per (batch*head, 16-column tile of the state); wave w owns state
// rows 16w..16w+15.  Each step is a dk x dk by dk x 16 product on
// v_mfma_f32_16x16x32_bf16 with both operands split into bf16 high and low parts
// (hi*hi + hi*lo + lo*hi, fp32 accumulation: about 16 mantissa bits), started from
// S_loc_i in the accumulator.
//
// The step chain is latency-bound, so nothing but the product sits on it:
//   * M_i arrives already split (the segment pass writes its high and low bf16
//     planes) and each wave keeps the rows of the next SCAN_DEPTH transitions in
//     flight in registers;
//   * the new start state is split once, by the wave that produced it, into
//     transposed bf16 high / low copies in LDS that every wave reads as its MFMA
//     B operand with 16-byte loads;
//   * one extra wave copies each start state (an fp32 copy in LDS) to HBM, so the
//     product waves issue only loads.
// starts[0] receives a copy of S0 (or zeros), so the pass that follows never reads
// S0 itself (S0 may alias the final state).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

constexpr int SCAN_DEPTH = 3;   // transitions in flight per wave

template <int DK>
__global__ __launch_bounds__(64 * (DK / 16 + 1)) void scan_kernel(ScanArgs a) {
    constexpr int NW = DK / 16;                   // product waves: one 16-row tile of the state each
    constexpr int KSTEP = (DK + 31) / 32;         // 32-deep MFMA steps over the contraction
    constexpr int LDB = 32 * KSTEP + 8;           // bf16 pitch of the transposed split copies
    constexpr int LDF = DK + 4;                   // fp32 pitch of the transposed copy (store wave)
    constexpr int D = SCAN_DEPTH;
    __shared__ __attribute__((aligned(16))) bf16 s_hi[16 * LDB];
    __shared__ __attribute__((aligned(16))) bf16 s_lo[16 * LDB];
    __shared__ __attribute__((aligned(16))) float s_f[16 * LDF];

    // The column tiles of one (batch, head) are 8 block indices apart, so they run on one
    // XCD (workgroups go round-robin over the 8 XCDs) and share its L2 copy of M_i.
    const int nblk = a.dv / 16;
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
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m = lane & 15, g = lane >> 4;
    const int col = 16 * jb + m;                  // state column of this lane (B / C layouts)
    const int row0 = 16 * w;
    const bool storer = w == NW;

    // contraction rows past DK (DK = 16) must read as zeros
    for (int i = threadIdx.x; i < 16 * LDB; i += 64 * (NW + 1)) {
        s_hi[i] = (bf16)0.f;
        s_lo[i] = (bf16)0.f;
    }
    __syncthreads();

    // publish rows row0 + 4g .. +3 of column m: fp32 for the store wave, split bf16 for the products
    auto put = [&](const f32x4& x) {
        *reinterpret_cast<f32x4*>(s_f + m * LDF + row0 + 4 * g) = x;
        bf16x4 hi, lo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            hi[j] = (bf16)x[j];
            lo[j] = (bf16)(x[j] - (float)hi[j]);
        }
        *reinterpret_cast<bf16x4*>(s_hi + m * LDB + row0 + 4 * g) = hi;
        *reinterpret_cast<bf16x4*>(s_lo + m * LDB + row0 + 4 * g) = lo;
    };

    // the store wave writes start state i (in s_f) to starts[i]; rows spread over lanes
    auto store_start = [&](int i) {
        float* dst = a.starts + (bh * P + i) * DK * dv + 16 * jb;
#pragma unroll
        for (int it = 0; it < DK / 16; ++it) {                    // (row, column quad) pairs
            const int e = lane + 64 * it, row = e >> 2, cq = e & 3;
            f32x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = s_f[(4 * cq + j) * LDF + row];
            *reinterpret_cast<f32x4*>(dst + (int64_t)row * dv + 4 * cq) = v;
        }
    };

    if (!storer) {
        f32x4 cur;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            cur[r] = a.s0 ? a.s0[bh * DK * dv + (int64_t)(row0 + 4 * g + r) * dv + col] : 0.f;
        put(cur);
    }

    // transition rows of step i into slot u: lane (m, g) holds the high and low parts of
    // M_i[row0 + m][32 s + 8 g .. + 7]; S_loc_i rows row0 + 4 g + r of column col
    const bf16* mt = reinterpret_cast<const bf16*>(a.m_tr);    // [B*H][P][2][DK][DK]
    bf16x8 mh[D][KSTEP], ml[D][KSTEP];
    f32x4 sl[D];
    auto load_step = [&](int i, bf16x8 (&h)[KSTEP], bf16x8 (&l)[KSTEP], f32x4& s) {
        const bf16* Mh = mt + ((bh * P + i) * 2) * DK * DK + (int64_t)(row0 + m) * DK;
        const bf16* Ml = Mh + DK * DK;
#pragma unroll
        for (int t = 0; t < KSTEP; ++t) {
            const int k0 = 32 * t + 8 * g;
            if (k0 < DK) {
                h[t] = *reinterpret_cast<const bf16x8*>(Mh + k0);
                l[t] = *reinterpret_cast<const bf16x8*>(Ml + k0);
            } else {
#pragma unroll
                for (int j = 0; j < 8; ++j) h[t][j] = l[t][j] = (bf16)0.f;
            }
        }
        const float* L = a.s_loc + (bh * P + i) * DK * dv;
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] = L[(int64_t)(row0 + 4 * g + r) * dv + col];
    };
    const int nsteps = P - 1;
    if (nsteps > 0 && !storer) {
#pragma unroll
        for (int u = 0; u < D; ++u) load_step(min(u, nsteps - 1), mh[u], ml[u], sl[u]);
    }

    // The store wave and the product waves run separate loops with the same barriers, so the
    // product loop holds loads only and its memory counter waits cover exactly one slot.
    if (storer) {
        for (int i = 0; i < nsteps; ++i) {
            __syncthreads();                      // LDS holds the start of segment i
            store_start(i);
            __syncthreads();
        }
        __syncthreads();
        store_start(P - 1);
        return;
    }
    // one step: the start of segment i (in LDS) times M_i plus S_loc_i, from slot u
    auto step = [&](int i, int u, bool refill) {
        __syncthreads();                          // LDS holds the start of segment i
        f32x4 acc = sl[u], acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KSTEP; ++t) {
            const bf16x8 bh8 = *reinterpret_cast<const bf16x8*>(s_hi + m * LDB + 32 * t + 8 * g);
            const bf16x8 bl8 = *reinterpret_cast<const bf16x8*>(s_lo + m * LDB + 32 * t + 8 * g);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mh[u][t], bh8, acc, 0, 0, 0);
            acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mh[u][t], bl8, acc2, 0, 0, 0);
            acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ml[u][t], bh8, acc2, 0, 0, 0);
        }
        // the slot's registers are consumed: refill it with step i + D (clamped)
        if (refill) load_step(min(i + D, nsteps - 1), mh[u], ml[u], sl[u]);
        __syncthreads();                          // every wave has read the start of segment i
        put(acc + acc2);
    };
    // Whole groups of D steps per iteration, so every slot keeps its registers across the
    // back edge and the loop is entered only with the slots in load order; the last
    // nsteps % D steps follow it.
    int i = 0;
    for (; i + D <= nsteps; i += D) {
#pragma unroll
        for (int u = 0; u < D; ++u) step(i + u, u, true);
    }
#pragma unroll
    for (int u = 0; u < D - 1; ++u)
        if (i + u < nsteps) step(i + u, u, false);
    __syncthreads();
}

template <int DK>
static hipError_t launch_scan_dk(const ScanArgs& a, hipStream_t st) {
    const unsigned nblk = (unsigned)(a.B * a.H * (a.dv / 16));
    hipLaunchKernelGGL((scan_kernel<DK>), dim3(nblk), dim3(64 * (DK / 16 + 1)), 0, st, a);
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
