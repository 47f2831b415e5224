// Chunked KDA prefill for gfx950: one fused kernel per launch.
//
// Each workgroup owns one (batch, head, segment, column block) and walks its
// chunks of C tokens in order.  Per chunk, with Gamma the inclusive cumulative
// sum of the floored log-decay g and S the start state:
//
//   U  = (I + Diag(beta) A)^-1 Diag(beta) (V - (k e^Gamma) S)          (WY/UT form)
//   O  = (q e^Gamma) S + M U
//   S' = Diag(e^Gamma_C) S + (k e^(Gamma_C - Gamma))^T U
//   A[t,s] = sum_c k_tc k_sc e^(Gamma_tc - Gamma_sc)  (s < t),  M likewise with q (s <= t)
//
// Chunked evaluation has to divide by a cumulative decay; the floor on the
// log-decay bounds a 16-token tile's cumulative log-decay to [-80, 0], so its
// reciprocal stays below e^80 ~ 5.5e34, inside bf16, and the diagonal tiles
// can run as the same dense matrix products as every other tile (orkas.ai
// "Kimi K3 architecture", section "The floor that removed a GPU code path").
//
// Sub-tile factorisation used here.  Let t lie in 16-token sub-tile p of the
// chunk, gamma_t the inclusive cumulative log-decay inside that sub-tile
// (in [-80, 0]), tot_p its total and r_p = tot_0 + ... + tot_{p-1}.  Then
//   k_t e^Gamma_t           = [k_t e^gamma_t] e^r_p                (KL, <= 1)
//   e^(Gamma_t - Gamma_s)   = [e^gamma_t] f_pp' [e^(tot_p' - gamma_s)]
// with f_pp = e^-tot_p (<= e^80, the diagonal tile) and f_pp' = e^(r_p -
// r_p'+1) (<= 1) for p' < p.  So A and M tiles are (KL or QL) Diag(f) RH^T
// with both stored operands bounded by 1; the per-channel factor f is applied
// to the left operand in registers.  e^r_p is folded into the state operand:
// (k e^Gamma) S = KL (Diag(e^r_p) S).
//
// Matrix products run on MFMA: v_mfma_f32_16x16x32_bf16 for bf16 inputs,
// v_mfma_f32_16x16x4_f32 for float32 inputs.  The state stays in fp32 MFMA
// accumulators for the whole sequence; each wave owns 16 state columns
// (the recurrence is independent per column).  MFMA outputs (V - X, U) feed
// the next MFMA straight from registers: the contraction index of the next
// product is taken in the order the accumulator layout holds it, and the
// other operand is loaded from LDS in that same order ("chained" order).
// The triangular solve runs in fp32 (diagonal 16x16 blocks by forward
// substitution, off-diagonal blocks level by level).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// ---------------------------------------------------------------- MFMA operand policies
// Accumulator layout (both instructions): lane l holds C[4*(l/16) + r][l % 16], r = 0..3.
template <typename OpT> struct Mf;

template <> struct Mf<bf16> {
    static constexpr int KS = 32;          // contraction length per instruction
    typedef bf16x8 frag;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // natural order: lane (m = l%16, g = l/16) holds X[r0 + m][k0 + 8g + j], j < 8
    static __device__ __forceinline__ frag ld_nat(const bf16* X, int ld, int r0, int k0, int lane) {
        return *reinterpret_cast<const frag*>(X + (r0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
    }
    // chained order for step s: slot j<4 -> k = 32s + 4g + j, slot 4+j -> k = 32s + 16 + 4g + j,
    // i.e. rows 4g..4g+3 of accumulator tiles 2s and 2s+1
    static __device__ __forceinline__ frag ld_chain(const bf16* X, int ld, int r0, int s, int lane) {
        const bf16* p = X + (r0 + (lane & 15)) * ld + 32 * s + 4 * (lane >> 4);
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    template <int NTILE>
    static __device__ __forceinline__ frag b_chain(const f32x4 (&t)[NTILE], int s) {
        frag f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[j] = (bf16)(2 * s < NTILE ? t[2 * s][j] : 0.f);
            f[4 + j] = (bf16)(2 * s + 1 < NTILE ? t[2 * s + 1][j] : 0.f);
        }
        return f;
    }
    // scale a natural-order fragment by per-k factors fac[k0 + 8g + j]
    static __device__ __forceinline__ frag scale_nat(frag a, const float* fac, int k0, int lane) {
        const f32x4* f4 = reinterpret_cast<const f32x4*>(fac + k0 + 8 * (lane >> 4));
        const f32x4 lo = f4[0], hi = f4[1];
        frag r;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            r[j] = (bf16)((float)a[j] * lo[j]);
            r[4 + j] = (bf16)((float)a[4 + j] * hi[j]);
        }
        return r;
    }
    static constexpr int steps(int K) { return (K + KS - 1) / KS; }
};

template <> struct Mf<float> {
    static constexpr int KS = 4;
    typedef float frag;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    // natural order: lane (m, g) holds X[r0 + m][k0 + g]
    static __device__ __forceinline__ frag ld_nat(const float* X, int ld, int r0, int k0, int lane) {
        return X[(r0 + (lane & 15)) * ld + k0 + (lane >> 4)];
    }
    // chained order for step s: k = 16*(s/4) + 4g + s%4, i.e. row 4g + s%4 of accumulator tile s/4
    static __device__ __forceinline__ frag ld_chain(const float* X, int ld, int r0, int s, int lane) {
        return X[(r0 + (lane & 15)) * ld + 16 * (s >> 2) + 4 * (lane >> 4) + (s & 3)];
    }
    template <int NTILE>
    static __device__ __forceinline__ frag b_chain(const f32x4 (&t)[NTILE], int s) {
        return t[s >> 2][s & 3];
    }
    static __device__ __forceinline__ frag scale_nat(frag a, const float* fac, int k0, int lane) {
        return a * fac[k0 + (lane >> 4)];
    }
    static constexpr int steps(int K) { return K / KS; }
};

// ---------------------------------------------------------------- LDS layout
struct Lds {
    int kl, ql, rh, tinv, kht, abuf, tb, mb, vb, lp;
    int tot, rr, er, fp, fd, fo, egc, beta, total;
};

__host__ __device__ constexpr int align16(int x) { return (x + 15) & ~15; }

// E: bytes per operand element; KS: MFMA contraction length
__host__ __device__ constexpr Lds lds_layout(int E, int KS, int DK, int C, int DVB) {
    const int PADE = 16 / E;
    const int NT = C / 16;
    const int LDK = (DK > KS ? DK : KS) + PADE;
    const int LC = (C > KS ? C : KS) + PADE;
    const int LCA = C + 4;
    const int LV = DVB + PADE;
    const int FK = DK > KS ? DK : KS;          // factor row length (padded for DK < KS)
    const int NPAIR = NT * (NT - 1) / 2;
    Lds L{};
    int off = 0;
    L.kl = off;   off += align16(C * LDK * E);
    L.ql = off;   off += align16(C * LDK * E);
    L.rh = off;   L.tinv = off;
    {
        const int a = align16(C * LDK * E), b = align16(C * LCA * 4);
        off += a > b ? a : b;
    }
    L.kht = off;  off += align16(FK * LC * E);
    L.abuf = off; off += align16(C * LCA * 4);
    L.tb = off;   off += align16(C * LC * E);
    L.mb = off;   off += align16(C * LC * E);
    L.vb = off;   off += align16(C * LV * E);
    L.lp = off;   off += align16((NPAIR > 0 ? NPAIR : 1) * 256 * 4);
    L.tot = off;  off += align16(NT * FK * 4);
    L.rr = off;   off += align16((NT + 1) * FK * 4);
    L.er = off;   off += align16(NT * FK * 4);
    L.fp = off;   off += align16(NT * FK * 4);
    L.fd = off;   off += align16(NT * FK * 4);
    L.fo = off;   off += align16((NPAIR > 0 ? NPAIR : 1) * FK * 4);
    L.egc = off;  off += align16(FK * 4);
    L.beta = off; off += align16(C * 4);
    L.total = off;
    return L;
}

__device__ __forceinline__ int pair_index(int p, int pp) { return p * (p - 1) / 2 + pp; }   // pp < p

// store 16 consecutive values (converted) at dst (16-byte aligned)
__device__ __forceinline__ void store16(bf16* dst, const float (&x)[16]) {
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (bf16)x[j];
        b[j] = (bf16)x[8 + j];
    }
    reinterpret_cast<bf16x8*>(dst)[0] = a;
    reinterpret_cast<bf16x8*>(dst)[1] = b;
}
__device__ __forceinline__ void store16(float* dst, const float (&x)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
        reinterpret_cast<f32x4*>(dst)[j] = f32x4{x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]};
}

__device__ __forceinline__ void load_pair(const bf16* p, float& x, float& y) {
    const bf16x2 v = *reinterpret_cast<const bf16x2*>(p);
    x = (float)v[0];
    y = (float)v[1];
}
__device__ __forceinline__ void load_pair(const float* p, float& x, float& y) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    x = v.x;
    y = v.y;
}
__device__ __forceinline__ void store_pair(bf16* p, float x, float y) {
    *reinterpret_cast<bf16x2*>(p) = bf16x2{(bf16)x, (bf16)y};
}
__device__ __forceinline__ void store_pair(float* p, float x, float y) {
    *reinterpret_cast<float2*>(p) = make_float2(x, y);
}

// ---------------------------------------------------------------- the kernel
// MODE 0: outputs and final states; MODE 1: segment summaries (see ChunkArgs).
template <typename OpT, int DK, int C, int MODE>
__global__ __launch_bounds__(512) void chunk_kernel(ChunkArgs a) {
    using MF = Mf<OpT>;
    using frag = typename MF::frag;
    constexpr int E = sizeof(OpT);
    constexpr int KS = MF::KS;
    constexpr int PADE = 16 / E;
    constexpr int NT = C / 16;                       // 16-token sub-tiles per chunk
    constexpr int NCT = DK / 16;                     // 16-row tiles of the state
    constexpr int LDK = (DK > KS ? DK : KS) + PADE;
    constexpr int LC = (C > KS ? C : KS) + PADE;
    constexpr int LCA = C + 4;
    constexpr int FK = DK > KS ? DK : KS;
    constexpr int NPAIR = NT * (NT - 1) / 2;
    constexpr int SK_DK = MF::steps(DK);             // MFMA steps over the key dimension
    constexpr int SK_C = MF::steps(C);               // MFMA steps over the chunk

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int NTH = blockDim.x;
    const int DVB = a.dv_block;
    const int LV = DVB + PADE;
    const Lds L = lds_layout(E, KS, DK, C, DVB);
    OpT* s_kl = reinterpret_cast<OpT*>(smem + L.kl);
    OpT* s_ql = reinterpret_cast<OpT*>(smem + L.ql);
    OpT* s_rh = reinterpret_cast<OpT*>(smem + L.rh);
    float* s_tinv = reinterpret_cast<float*>(smem + L.tinv);
    OpT* s_kht = reinterpret_cast<OpT*>(smem + L.kht);
    float* s_abuf = reinterpret_cast<float*>(smem + L.abuf);
    OpT* s_tb = reinterpret_cast<OpT*>(smem + L.tb);
    OpT* s_mb = reinterpret_cast<OpT*>(smem + L.mb);
    OpT* s_vb = reinterpret_cast<OpT*>(smem + L.vb);
    float* s_lp = reinterpret_cast<float*>(smem + L.lp);
    float* s_tot = reinterpret_cast<float*>(smem + L.tot);
    float* s_rr = reinterpret_cast<float*>(smem + L.rr);
    float* s_er = reinterpret_cast<float*>(smem + L.er);
    float* s_fp = reinterpret_cast<float*>(smem + L.fp);
    float* s_fd = reinterpret_cast<float*>(smem + L.fd);
    float* s_fo = reinterpret_cast<float*>(smem + L.fo);
    float* s_egc = reinterpret_cast<float*>(smem + L.egc);
    float* s_beta = reinterpret_cast<float*>(smem + L.beta);

    // ---- which (batch, head, segment, column block) this workgroup owns
    const int H = a.H, dv = a.dv;
    const int ncols = MODE == 0 ? dv : dv + DK;
    const int ncb = ncols / DVB;
    const int nseg_grid = MODE == 0 ? a.n_seg : a.n_seg - 1;
    int64_t bid = blockIdx.x;
    const int cb = (int)(bid % ncb);
    bid /= ncb;
    const int seg = (int)(bid % nseg_grid);
    bid /= nseg_grid;
    const int h = (int)(bid % H);
    const int64_t b = bid / H;
    const int64_t bh = b * H + h;
    const int64_t T = a.T;
    const int64_t t_begin = (int64_t)seg * a.seg_len;
    const int64_t t_end = t_begin + a.seg_len < T ? t_begin + a.seg_len : T;

    const int colw = cb * DVB + 16 * wave;           // first (virtual) column of this wave
    const bool mcols = MODE == 1 && colw >= dv;    // wave holds transition columns
    const bool blk_mcols = MODE == 1 && cb * DVB >= dv;
    const bool want_o = MODE == 0;
    const int g4 = 4 * (lane >> 4), jl = lane & 15;

    const OpT* gq = reinterpret_cast<const OpT*>(a.q);
    const OpT* gk = reinterpret_cast<const OpT*>(a.k);
    const OpT* gv = reinterpret_cast<const OpT*>(a.v);
    OpT* go = reinterpret_cast<OpT*>(a.o);

    // ---- zero all LDS once: padding columns and the upper blocks of T and M stay zero
    for (int i = tid * 16; i < L.total; i += NTH * 16)
        *reinterpret_cast<f32x4*>(smem + i) = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- start state into accumulator layout: Sacc[tau][r] = S[16 tau + g4 + r][colw + jl]
    f32x4 Sacc[NCT];
    {
        const float* src = nullptr;
        int64_t ld = dv;
        int col = colw + jl;
        if (MODE == 0) {
            // with segments every start (segment 0's included) comes from the scan's
            // output, so S0 is never read here while another workgroup writes S_T
            if (a.n_seg == 1) src = a.s0 ? a.s0 + bh * DK * dv : nullptr;
            else src = a.starts + (bh * a.n_seg + seg) * DK * dv;
        }
#pragma unroll
        for (int tau = 0; tau < NCT; ++tau)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * tau + g4 + r;
                float x = 0.f;
                if (src) x = src[row * ld + col];
                else if (mcols) x = (row == col - dv) ? 1.f : 0.f;
                Sacc[tau][r] = x;
            }
    }

    for (int64_t t0 = t_begin; t0 < t_end; t0 += C) {
        const int Tc = (int)(t_end - t0 < C ? t_end - t0 : C);
        __syncthreads();   // previous chunk's readers of LDS are done

        // ---- V block and beta into LDS (zeros past the end and for transition columns)
        {
            constexpr int VE = 16 / E;                 // elements per 16-byte vector
            const int vpr = DVB / VE;                  // vectors per row
            for (int i = tid; i < C * vpr; i += NTH) {
                const int t = i / vpr, cv = (i % vpr) * VE;
                f32x4 val = {0.f, 0.f, 0.f, 0.f};
                if (t < Tc && !blk_mcols)
                    val = *reinterpret_cast<const f32x4*>(gv + ((b * T + t0 + t) * H + h) * dv + cb * DVB + cv);
                *reinterpret_cast<f32x4*>(s_vb + t * LV + cv) = val;
            }
            for (int t = tid; t < C; t += NTH)
                s_beta[t] = t < Tc ? a.beta[(b * T + t0 + t) * H + h] : 0.f;
        }

        // ---- gate prep: one item = (channel pair, sub-tile); cumulative log-decay inside
        // the sub-tile, scaled operands KL = k e^gamma, QL = q e^gamma, RH = k e^(tot-gamma)
        for (int it = tid; it < (DK / 2) * NT; it += NTH) {
            const int c = 2 * (it % (DK / 2)), p = it / (DK / 2);
            float ga[16][2], kk[16][2], qq[16][2];
            float g0 = 0.f, g1 = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int t = 16 * p + i;
                float la0 = 0.f, la1 = 0.f;
                kk[i][0] = kk[i][1] = qq[i][0] = qq[i][1] = 0.f;
                if (t < Tc) {
                    const int64_t base = ((b * T + t0 + t) * H + h) * DK + c;
                    load_pair(a.log_alpha + base, la0, la1);
                    load_pair(gk + base, kk[i][0], kk[i][1]);
                    load_pair(gq + base, qq[i][0], qq[i][1]);
                }
                g0 += clamp_log_alpha(la0);
                g1 += clamp_log_alpha(la1);
                ga[i][0] = g0;
                ga[i][1] = g1;
            }
            float h0[16], h1[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int t = 16 * p + i;
                const float a0 = fast_exp(ga[i][0]), a1 = fast_exp(ga[i][1]);
                const float c0 = fast_exp(g0 - ga[i][0]), c1 = fast_exp(g1 - ga[i][1]);
                store_pair(s_kl + t * LDK + c, kk[i][0] * a0, kk[i][1] * a1);
                store_pair(s_ql + t * LDK + c, qq[i][0] * a0, qq[i][1] * a1);
                store_pair(s_rh + t * LDK + c, kk[i][0] * c0, kk[i][1] * c1);
                h0[i] = kk[i][0] * c0;
                h1[i] = kk[i][1] * c1;
            }
            store16(s_kht + c * LC + 16 * p, h0);
            store16(s_kht + (c + 1) * LC + 16 * p, h1);
            s_tot[p * FK + c] = g0;
            s_tot[p * FK + c + 1] = g1;
        }
        __syncthreads();

        // ---- per-channel factors
        for (int c = tid; c < DK; c += NTH) {
            float r = 0.f;
            s_rr[c] = 0.f;
#pragma unroll
            for (int p = 0; p < NT; ++p) {
                const float tot = s_tot[p * FK + c];
                s_er[p * FK + c] = fast_exp(r);
                s_fd[p * FK + c] = fast_exp(-tot);
                r += tot;
                s_rr[(p + 1) * FK + c] = r;
            }
            s_egc[c] = fast_exp(r);
#pragma unroll
            for (int p = 0; p < NT; ++p) {
                s_fp[p * FK + c] = fast_exp(r - s_rr[(p + 1) * FK + c]);
#pragma unroll
                for (int pp = 0; pp < p; ++pp)
                    s_fo[pair_index(p, pp) * FK + c] = fast_exp(s_rr[p * FK + c] - s_rr[(pp + 1) * FK + c]);
            }
        }
        __syncthreads();

        // ---- K-hat^T = (k e^(tot_p - gamma))^T scaled by e^(Gamma_C - r_{p+1})
        for (int i = tid; i < DK * C; i += NTH) {
            const int c = i / C, t = i % C;
            OpT* p = s_kht + c * LC + t;
            *p = from_f32<OpT>(to_f32(*p) * s_fp[(t / 16) * FK + c]);
        }
        // ---- A (beta-scaled, strictly lower) and M (lower) tiles on MFMA
        {
            constexpr int NTASK = NT * (NT + 1);
            for (int task = wave; task < NTASK; task += NTH / 64) {
                if (!want_o && (task & 1)) continue;            // M only needed for outputs
                const bool isM = task & 1;
                int pr = task >> 1, p = 0;
                while (pr > p) { pr -= p + 1; ++p; }
                const int pp = pr;                                // pp <= p
                const OpT* left = isM ? s_ql : s_kl;
                const float* fac = p == pp ? s_fd + p * FK
                                 : (p > pp + 1 ? s_fo + pair_index(p, pp) * FK : nullptr);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < SK_DK; ++ks) {
                    frag af = MF::ld_nat(left, LDK, 16 * p, ks * KS, lane);
                    if (fac) af = MF::scale_nat(af, fac, ks * KS, lane);
                    const frag bf = MF::ld_nat(s_rh, LDK, 16 * pp, ks * KS, lane);
                    acc = MF::mma(af, bf, acc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tr = g4 + r;                        // row within tile
                    const int t = 16 * p + tr, s = 16 * pp + jl;
                    if (!isM) {
                        float val = acc[r] * s_beta[t];
                        if (p == pp && jl >= tr) val = 0.f;
                        s_abuf[t * LCA + s] = val;
                    } else {
                        float val = acc[r];
                        if (p == pp && jl > tr) val = 0.f;
                        s_mb[t * LC + s] = from_f32<OpT>(val);
                    }
                }
            }
        }
        __syncthreads();

        // ---- T = (I + Diag(beta) A)^-1 Diag(beta), fp32.  Diagonal blocks first.
        if (tid < NT * 16) {
            const int p = tid >> 4, j = tid & 15;
            float x[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float acc = (t == j) ? 1.f : 0.f;
                const float* row = s_abuf + (16 * p + t) * LCA + 16 * p;
#pragma unroll
                for (int s = 0; s < t; ++s) acc -= row[s] * x[s];
                x[t] = acc;
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) s_tinv[(16 * p + t) * LCA + 16 * p + j] = x[t];
        }
        __syncthreads();
        if constexpr (NT > 1) {
            // L'_pq = N_pp L_pq for p > q (N_pp = inverse of the diagonal block)
            for (int it = tid; it < NPAIR * 256; it += NTH) {
                const int pr = it >> 8, i = (it >> 4) & 15, j = it & 15;
                int p = 1, q = pr;
                while (q >= p) { q -= p; ++p; }
                const float* nrow = s_tinv + (16 * p + i) * LCA + 16 * p;
                const float* lcol = s_abuf + (16 * p) * LCA + 16 * q + j;
                float acc = 0.f;
#pragma unroll
                for (int u = 0; u < 16; ++u) acc += nrow[u] * lcol[u * LCA];
                s_lp[it] = acc;
            }
            __syncthreads();
            // X_pq = -sum_{m=q}^{p-1} L'_pm X_mq, level by level (X_qq = N_qq)
#pragma unroll
            for (int d = 1; d < NT; ++d) {
                for (int it = tid; it < (NT - d) * 256; it += NTH) {
                    const int q = it >> 8, i = (it >> 4) & 15, j = it & 15;
                    const int p = q + d;
                    float acc = 0.f;
                    for (int m = q; m < p; ++m) {
                        const float* lrow = s_lp + pair_index(p, m) * 256 + i * 16;
                        const float* xcol = s_tinv + (16 * m) * LCA + 16 * q + j;
#pragma unroll
                        for (int u = 0; u < 16; ++u) acc += lrow[u] * xcol[u * LCA];
                    }
                    s_tinv[(16 * p + i) * LCA + 16 * q + j] = -acc;
                }
                __syncthreads();
            }
        }
        // T = Tinv Diag(beta) on the lower block triangle (upper blocks stay zero)
        for (int i = tid; i < C * C; i += NTH) {
            const int t = i / C, s = i % C;
            if (s < 16 * (t / 16 + 1)) s_tb[t * LC + s] = from_f32<OpT>(s_tinv[t * LCA + s] * s_beta[s]);
        }
        __syncthreads();

        // ---- the state chain, per wave on its 16 columns
        {
            f32x4 X[NT], QS[NT];
#pragma unroll
            for (int p = 0; p < NT; ++p) {
                f32x4 sc[NCT];
#pragma unroll
                for (int tau = 0; tau < NCT; ++tau)
#pragma unroll
                    for (int r = 0; r < 4; ++r) sc[tau][r] = Sacc[tau][r] * s_er[p * FK + 16 * tau + g4 + r];
                X[p] = f32x4{0.f, 0.f, 0.f, 0.f};
                QS[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < SK_DK; ++s) {
                    const frag sf = MF::b_chain(sc, s);
                    X[p] = MF::mma(MF::ld_chain(s_kl, LDK, 16 * p, s, lane), sf, X[p]);
                    if (want_o) QS[p] = MF::mma(MF::ld_chain(s_ql, LDK, 16 * p, s, lane), sf, QS[p]);
                }
            }
            // V' = V - X
            f32x4 Vp[NT];
#pragma unroll
            for (int p = 0; p < NT; ++p)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float vv = mcols ? 0.f : to_f32(s_vb[(16 * p + g4 + r) * LV + 16 * wave + jl]);
                    Vp[p][r] = vv - X[p][r];
                }
            // U = T V'
            f32x4 U[NT];
#pragma unroll
            for (int p = 0; p < NT; ++p) {
                U[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < SK_C; ++s)
                    U[p] = MF::mma(MF::ld_chain(s_tb, LC, 16 * p, s, lane), MF::b_chain(Vp, s), U[p]);
            }
            // O = Q~ S + M U, staged in the V buffer (same wave, same columns)
            if (want_o) {
#pragma unroll
                for (int p = 0; p < NT; ++p) {
                    f32x4 O = QS[p];
#pragma unroll
                    for (int s = 0; s < SK_C; ++s)
                        O = MF::mma(MF::ld_chain(s_mb, LC, 16 * p, s, lane), MF::b_chain(U, s), O);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        s_vb[(16 * p + g4 + r) * LV + 16 * wave + jl] = from_f32<OpT>(O[r]);
                }
            }
            // S <- Diag(e^Gamma_C) S + K-hat^T U
#pragma unroll
            for (int tau = 0; tau < NCT; ++tau) {
#pragma unroll
                for (int r = 0; r < 4; ++r) Sacc[tau][r] *= s_egc[16 * tau + g4 + r];
#pragma unroll
                for (int s = 0; s < SK_C; ++s)
                    Sacc[tau] = MF::mma(MF::ld_chain(s_kht, LC, 16 * tau, s, lane), MF::b_chain(U, s), Sacc[tau]);
            }
        }
        __syncthreads();

        // ---- write the chunk's outputs
        if (want_o) {
            constexpr int VE = 16 / E;
            const int vpr = DVB / VE;
            for (int i = tid; i < Tc * vpr; i += NTH) {
                const int t = i / vpr, cv = (i % vpr) * VE;
                *reinterpret_cast<f32x4*>(go + ((b * T + t0 + t) * H + h) * dv + cb * DVB + cv) =
                    *reinterpret_cast<const f32x4*>(s_vb + t * LV + cv);
            }
        }
    }

    // ---- final state of this unit
    {
        float* dst = nullptr;
        int64_t ld = 0;
        int col = colw + jl;
        if (MODE == 0) {
            if (seg == a.n_seg - 1) { dst = a.s_final + bh * DK * dv; ld = dv; }
        } else if (!mcols) {
            dst = a.s_loc + (bh * a.n_seg + seg) * DK * dv; ld = dv;
        } else {
            dst = a.m_tr + (bh * a.n_seg + seg) * DK * DK; ld = DK; col -= dv;
        }
        if (dst) {
#pragma unroll
            for (int tau = 0; tau < NCT; ++tau)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(16 * tau + g4 + r) * ld + col] = Sacc[tau][r];
        }
    }
}

// ---------------------------------------------------------------- launch
size_t chunk_lds_bytes(bool bf16_, int dk, int chunk, int dv_block) {
    const int E = bf16_ ? 2 : 4, KS = bf16_ ? 32 : 4;
    return (size_t)lds_layout(E, KS, dk, chunk, dv_block).total;
}

template <typename OpT, int DK, int C, int MODE>
static hipError_t launch_chunk_m(const ChunkArgs& a, hipStream_t st) {
    const size_t lds = chunk_lds_bytes(sizeof(OpT) == 2, DK, C, a.dv_block);
    auto kern = chunk_kernel<OpT, DK, C, MODE>;
    static bool attr_set = false;   // per instantiation; the attribute is device-independent
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds > 65536 ? 163840 : 65536);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int ncols = a.mode == 0 ? a.dv : a.dv + DK;
    const int nseg_grid = a.mode == 0 ? a.n_seg : a.n_seg - 1;
    const int64_t nblk = a.B * a.H * (int64_t)nseg_grid * (ncols / a.dv_block);
    if (nblk <= 0) return hipSuccess;
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(64 * (a.dv_block / 16)), lds, st, a);
    return hipGetLastError();
}

template <typename OpT, int DK, int C>
static hipError_t launch_chunk_t(const ChunkArgs& a, hipStream_t st) {
    return a.mode == 0 ? launch_chunk_m<OpT, DK, C, 0>(a, st) : launch_chunk_m<OpT, DK, C, 1>(a, st);
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
