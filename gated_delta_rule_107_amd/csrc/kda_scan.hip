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
//     planes) and is copied from HBM straight into LDS (global_load_lds, 16 bytes
//     per lane) one step ahead, into the other of two buffers, with an XOR
//     swizzle of its 16-byte granules so that the A-operand reads are free of
//     bank conflicts; S_loc_i is prefetched into registers one step ahead;
//   * the new start state is split once, by the wave that produced it, into
//     transposed bf16 high / low copies in LDS that every wave reads as its MFMA
//     B operand with 16-byte loads;
//   * one extra wave copies each start state (an fp32 copy in LDS) to HBM, so the
//     product waves' memory counter only tracks their own loads.
// starts[0] receives a copy of S0 (or zeros), so the pass that follows never reads
// S0 itself (S0 may alias the final state).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// Workgroup barrier for LDS traffic only.  __syncthreads() also carries a workgroup
// release fence, which waits for every vector-memory operation in flight, the
// transition copy into LDS included; this barrier waits for this wave's own LDS
// accesses (lgkmcnt) and, in lds_vm_barrier, for its vector-memory operations.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void lds_vm_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int DK>
__global__ __launch_bounds__(64 * (DK / 16 + 1)) void scan_kernel(ScanArgs a) {
    constexpr int NW = DK / 16;                   // product waves: one 16-row tile of the state each
    constexpr int KSTEP = (DK + 31) / 32;         // 32-deep MFMA steps over the contraction
    constexpr int LDB = 32 * KSTEP + 8;           // bf16 pitch of the transposed split copies
    constexpr int LDF = DK + 4;                   // fp32 pitch of the transposed copy (store wave)
    constexpr int NG = DK / 8;                    // 16-byte granules per row of one plane
    constexpr int NGX = NG < 8 ? NG : 8;          // swizzle period
    constexpr int GM = 2 * DK * NG;               // granules of one transition (two planes)
    constexpr int NI = GM / 64 / NW;              // copy instructions per product wave
    static_assert(NI * 64 * NW == GM, "transition copy map");
    __shared__ __attribute__((aligned(16))) bf16 s_hi[16 * LDB];
    __shared__ __attribute__((aligned(16))) bf16 s_lo[16 * LDB];
    __shared__ __attribute__((aligned(16))) float s_f[16 * LDF];
    __shared__ bf16x8 s_m[2 * GM];                // two transition buffers, swizzled granules

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
    lds_barrier();

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

    // LDS granule q of a buffer holds granule c = (q % NG) ^ (r % NGX) of row r = (q / NG) % DK
    // of plane q / (DK NG); this lane copies granules (w NI + j) 64 + lane, j < NI
    const bf16* mt = reinterpret_cast<const bf16*>(a.m_tr);    // [B*H][P][2][DK][DK]
    unsigned src_off[NI];                                        // bf16 offsets inside one M_i
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int q = (w * NI + j) * 64 + lane;
        const int pl = q / (DK * NG), r = (q / NG) % DK, c = (q % NG) ^ (r % NGX);
        src_off[j] = (unsigned)((pl * DK + r) * DK + c * 8);
    }
    auto copy_m = [&](int i, int buf) {
        const bf16* M = mt + (bh * P + i) * 2 * DK * DK;
#pragma unroll
        for (int j = 0; j < NI; ++j)
            copy16_global_to_lds(M + src_off[j], s_m + buf * GM + (w * NI + j) * 64);
    };
    auto a_granule = [&](int buf, int pl, int r, int c) -> bf16x8 {
        return s_m[buf * GM + (pl * DK + r) * NG + (c ^ (r % NGX))];
    };
    f32x4 sl;
    auto load_sloc = [&](int i) {
        const float* L = a.s_loc + (bh * P + i) * DK * dv;
#pragma unroll
        for (int r = 0; r < 4; ++r) sl[r] = L[(int64_t)(row0 + 4 * g + r) * dv + col];
    };
    const int nsteps = P - 1;

    // The store wave and the product waves run separate loops with the same barriers.
    if (storer) {
        for (int i = 0; i < nsteps; ++i) {
            lds_barrier();                        // LDS holds the start of segment i
            store_start(i);
            lds_barrier();
        }
        lds_barrier();
        store_start(P - 1);
        return;
    }
    if (nsteps > 0) {
        copy_m(0, 0);
        load_sloc(0);
    }
    for (int i = 0; i < nsteps; ++i) {
        const int buf = i & 1;
        lds_vm_barrier();                         // every share of M_i landed; LDS holds start i
        // operands into registers first, then the next transition's copy into the other buffer
        bf16x8 ah[KSTEP], al[KSTEP], bh8[KSTEP], bl8[KSTEP];
#pragma unroll
        for (int t = 0; t < KSTEP; ++t) {
            const int c = 4 * t + g;
            const bool in = 8 * c < DK;
            const int r = row0 + m;
            ah[t] = in ? a_granule(buf, 0, r, c) : bf16x8{};
            al[t] = in ? a_granule(buf, 1, r, c) : bf16x8{};
            bh8[t] = *reinterpret_cast<const bf16x8*>(s_hi + m * LDB + 32 * t + 8 * g);
            bl8[t] = *reinterpret_cast<const bf16x8*>(s_lo + m * LDB + 32 * t + 8 * g);
        }
        const f32x4 acc0 = sl;
        if (i + 1 < nsteps) {
            copy_m(i + 1, buf ^ 1);
            load_sloc(i + 1);
        }
        f32x4 acc = acc0, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KSTEP; ++t) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[t], bh8[t], acc, 0, 0, 0);
            acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[t], bl8[t], acc2, 0, 0, 0);
            acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[t], bh8[t], acc2, 0, 0, 0);
        }
        lds_barrier();                            // every wave has read start i and M_i
        put(acc + acc2);
    }
    lds_barrier();
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
