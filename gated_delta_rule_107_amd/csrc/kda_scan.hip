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
//     planes); each wave loads its 16 rows of it from global memory straight into
//     registers in the MFMA's A-operand layout, one step ahead (the transitions do
//     not depend on the chain), so the transition costs no LDS traffic or space;
//     S_loc_i is prefetched into registers one step ahead;
//   * the new start state is split once, by the wave that produced it, into
//     transposed bf16 high / low copies in LDS that every wave reads as its MFMA
//     B operand with 16-byte loads; they are double-buffered, so a step needs one
//     barrier;
//   * one extra wave copies each start state (a row-major fp32 copy in LDS) to HBM,
//     so the product waves' memory counter only tracks their own loads.
// A step is bounded by the vector-memory path of the CU: each workgroup needs all of M_i
// (64 KiB, both planes) per step for its 16 columns.
// starts[0] receives a copy of S0 (or zeros), so the pass that follows never reads
// S0 itself (S0 may alias the final state).  In the lead form of a plan the chain starts
// at segment 1 from the start state the lead launch wrote (first = 1).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// Workgroup barrier for LDS traffic only.  __syncthreads() also carries a workgroup
// release fence, which waits for every vector-memory operation in flight, the transition
// loads of the next step included; this barrier waits for this wave's own LDS accesses
// (lgkmcnt) only.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <bool V> struct Set { static constexpr bool value = V; };

template <int DK>
__global__ __launch_bounds__(64 * (DK / 16 + 1)) void scan_kernel(ScanArgs a) {
    constexpr int NW = DK / 16;                   // product waves: one 16-row tile of the state each
    constexpr int KSTEP = (DK + 31) / 32;         // 32-deep MFMA steps over the contraction
    constexpr int LDB = 32 * KSTEP + 8;           // bf16 pitch of the transposed split copies
    constexpr int LDR = 20;                       // fp32 pitch of the row-major copy (store wave)
    // the start state of step i in buffer i & 1: split bf16 copies (transposed) for the
    // products, a row-major fp32 copy for the store wave
    __shared__ __attribute__((aligned(16))) bf16 s_hi[2][16 * LDB];
    __shared__ __attribute__((aligned(16))) bf16 s_lo[2][16 * LDB];
    __shared__ __attribute__((aligned(16))) float s_f[2][DK * LDR];

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
    // this (sequence, head)'s segments: P of them, pairs and starts at base + i
    int P = a.n_seg;
    int64_t base = bh * P;
    if (a.seq_table) {
        const int2 e = a.seq_table[bh / a.H];
        P = e.y;
        base = (bh % a.H) * (int64_t)a.n_seg + e.x;
    }
    // lead form: the chain starts at segment 1, whose start state the lead launch wrote
    P -= a.first;
    base += a.first;
    const int dv = a.dv;
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int m = lane & 15, g = lane >> 4;
    const int col = 16 * jb + m;                  // state column of this lane (B / C layouts)
    const int row0 = 16 * w;
    const bool storer = w == NW;

    // contraction rows past DK (DK = 16) must read as zeros
    for (int i = threadIdx.x; i < 2 * 16 * LDB; i += 64 * (NW + 1)) {
        (&s_hi[0][0])[i] = (bf16)0.f;
        (&s_lo[0][0])[i] = (bf16)0.f;
    }
    lds_barrier();

    // publish rows row0 + 4g .. +3 of column m into buffer b: fp32 for the store wave, split
    // bf16 for the products
    auto put = [&](const f32x4& x, int b) {
#pragma unroll
        for (int r = 0; r < 4; ++r) s_f[b][(row0 + 4 * g + r) * LDR + m] = x[r];
        bf16x4 hi, lo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            hi[j] = (bf16)x[j];
            lo[j] = (bf16)(x[j] - (float)hi[j]);
        }
        *reinterpret_cast<bf16x4*>(s_hi[b] + m * LDB + row0 + 4 * g) = hi;
        *reinterpret_cast<bf16x4*>(s_lo[b] + m * LDB + row0 + 4 * g) = lo;
    };

    // the store wave writes start state i (in s_f[i & 1]) to starts[i]: 16 bytes of a row
    // per lane, read as one piece from the row-major copy
    auto store_start = [&](int i) {
        const float* f = s_f[i & 1];
        float* dst = a.starts + (base + i) * DK * dv + 16 * jb;
        // every read first, then the stores: one LDS round trip per step, not one per store
        f32x4 v[DK / 16];
#pragma unroll
        for (int it = 0; it < DK / 16; ++it) {                    // (row, column quad) pairs
            const int e = lane + 64 * it, row = e >> 2, cq = e & 3;
            v[it] = *reinterpret_cast<const f32x4*>(f + row * LDR + 4 * cq);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int it = 0; it < DK / 16; ++it) {
            const int e = lane + 64 * it, row = e >> 2, cq = e & 3;
            *reinterpret_cast<f32x4*>(dst + (int64_t)row * dv + 4 * cq) = v[it];
        }
    };

    // One barrier per step: the start states are double-buffered, so step i's products read
    // buffer i & 1 while the new state goes to the other buffer, which every wave finished
    // reading before this step's barrier (and the store wave before it, too).
    const int nsteps = P - 1;
    if (storer) {
        for (int i = 0; i < P; ++i) {
            lds_barrier();                        // LDS holds the start of segment i
            if (i > 0 || !a.first) store_start(i);    // (a given start is not stored again)
        }
        return;
    }

    {
        // the chain's first start: S0 (or zeros), or in the lead form the given start state
        const float* s_in = a.first ? a.starts + base * DK * dv : (a.s0 ? a.s0 + bh * DK * dv : nullptr);
        f32x4 cur;
#pragma unroll
        for (int r = 0; r < 4; ++r) cur[r] = s_in ? s_in[(int64_t)(row0 + 4 * g + r) * dv + col] : 0.f;
        put(cur, 0);
    }

    // The A operand (this wave's 16 rows of M_i, high and low planes) goes from global memory
    // straight into registers in the MFMA's layout (one contiguous 1 KiB run per load, as pass
    // 1 stores the transitions in that order), one step ahead into the register set of i's
    // parity: every transition is known before the chain starts, and no LDS traffic or buffer
    // is spent on them.  The loads are issued on every step (the last transition is re-read
    // past the end), so the compiler counts them exactly and a step waits only for the loads
    // of the step before (a load under a branch makes it wait for all of them).
    const bf16* mt = reinterpret_cast<const bf16*>(a.m_tr);    // [B*H][P][2][DK^2], mtr_index order
    bf16x8 ma0[2][KSTEP], ma1[2][KSTEP];                        // [plane][step] of M_i: even / odd i
    f32x4 sl0, sl1;                                             // S_loc_i: even / odd i
    auto load_m = [&](int i, bf16x8 (&dst)[2][KSTEP]) {
        const bf16* M = mt + (base + i) * 2 * DK * DK;
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
#pragma unroll
            for (int t = 0; t < KSTEP; ++t) {
                const int k0 = 32 * t + 8 * g;
                dst[pl][t] = k0 < DK ? *reinterpret_cast<const bf16x8*>(M + pl * DK * DK + mtr_index(DK, row0 + m, k0))
                                     : bf16x8{};
            }
    };
    auto load_sloc = [&](int i, f32x4& dst) {
        const float* L = a.s_loc + (base + i) * DK * dv;          // sloc_index order
        dst = *reinterpret_cast<const f32x4*>(L + sloc_index(DK, row0 + 4 * g, col));
    };
    if (nsteps > 0) {
        load_m(0, ma0);
        load_sloc(0, sl0);
    }
    auto step = [&](int i, auto odd_c) {
        constexpr bool odd = decltype(odd_c)::value;
        const int b = odd ? 1 : 0;
        lds_barrier();                            // LDS holds start i in buffer b
        // the next step's loads first (kept here by the scheduling barrier: the scheduler would
        // otherwise sink them below this step's products), then this step's B operands
        const int nx = i + 1 < nsteps ? i + 1 : nsteps - 1;
        if (odd) { load_m(nx, ma0); load_sloc(nx, sl0); }
        else { load_m(nx, ma1); load_sloc(nx, sl1); }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 bh8[KSTEP], bl8[KSTEP];
#pragma unroll
        for (int t = 0; t < KSTEP; ++t) {
            bh8[t] = *reinterpret_cast<const bf16x8*>(s_hi[b] + m * LDB + 32 * t + 8 * g);
            bl8[t] = *reinterpret_cast<const bf16x8*>(s_lo[b] + m * LDB + 32 * t + 8 * g);
        }
        const bf16x8 (&ma)[2][KSTEP] = odd ? ma1 : ma0;
        // hi*hi, hi*lo and lo*hi in three independent accumulator chains (the dependent chain
        // is the step's latency)
        f32x4 acc = odd ? sl1 : sl0, acc2 = {0.f, 0.f, 0.f, 0.f}, acc3 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < KSTEP; ++t) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ma[0][t], bh8[t], acc, 0, 0, 0);
            acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ma[0][t], bl8[t], acc2, 0, 0, 0);
            acc3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ma[1][t], bh8[t], acc3, 0, 0, 0);
        }
        put(acc + (acc2 + acc3), b ^ 1);
    };
    int i = 0;
    for (; i + 1 < nsteps; i += 2) {
        step(i, Set<false>{});
        step(i + 1, Set<true>{});
    }
    if (i < nsteps) step(i, Set<false>{});
    lds_barrier();                                // the last start is in LDS for the store wave
}

// Segment tables of packed sequences: one wave walks the sequences 64 at a time.  A sequence's
// range starts no earlier than the previous one's end (clamped into [0, T]), so the segments
// of any offsets array, valid or not, fit the n_slots >= ceil(T / seg_len) + n_seqs entries.
__global__ __launch_bounds__(64) void seg_table_kernel(SegTableArgs a) {
    const int lane = threadIdx.x;
    int64_t prev_end = 0;                        // end of the sequence before this group of 64
    int g0 = 0;                                  // first slot of this group's first sequence
    for (int i0 = 0; i0 < a.n_seqs; i0 += 64) {
        const int i = i0 + lane;
        const bool on = i < a.n_seqs;
        int64_t c0 = on ? a.cu_seqlens[i] : a.T, c1 = on ? a.cu_seqlens[i + 1] : a.T;
        c1 = c1 < 0 ? 0 : (c1 > a.T ? a.T : c1);
        c0 = c0 < 0 ? 0 : (c0 > a.T ? a.T : c0);
        if (c1 < c0) c1 = c0;
        // monotone ends: end_i = max over j <= i of c1_j (inclusive scan of maxima); begin_i =
        // max(c0_i, end_{i-1})
        int64_t end = c1;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int64_t o = __shfl_up(end, d, 64);
            if (lane >= d && o > end) end = o;
        }
        if (prev_end > end) end = prev_end;
        int64_t before = __shfl_up(end, 1, 64);
        if (lane == 0) before = prev_end;
        const int64_t beg = c0 > before ? (c0 < end ? c0 : end) : before;
        const int64_t len = end - beg;
        const int cnt = on ? (int)(len > 0 ? (len + a.seg_len - 1) / a.seg_len : 1) : 0;
        // exclusive scan of the counts
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d, 64);
            if (lane >= d) incl += o;
        }
        const int first = g0 + incl - cnt;
        if (on) {
            a.seq_table[i] = make_int2(first, cnt);
            for (int j = 0; j < cnt; ++j) {
                const int64_t tb = beg + (int64_t)j * a.seg_len;
                const int64_t te = tb + a.seg_len < end ? tb + a.seg_len : end;
                const int flags = (j == 0 ? SEG_FIRST : 0) | (j == cnt - 1 ? SEG_LAST : 0);
                if (first + j < a.n_slots) a.seg_table[first + j] = make_int4(i, (int)tb, (int)te, flags);
            }
        }
        g0 += __shfl(incl, 63, 64);
        prev_end = __shfl(end, 63, 64);
    }
    for (int g = g0 + lane; g < a.n_slots; g += 64) a.seg_table[g] = make_int4(-1, 0, 0, 0);
}

hipError_t launch_seg_table(const SegTableArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(seg_table_kernel, dim3(1), dim3(64), 0, st, a);
    return hipGetLastError();
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
