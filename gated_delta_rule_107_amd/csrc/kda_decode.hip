// Recurrent decode: one token per sequence with the state updated in place, and the
// multi-token verify / commit pair of speculative decoding built on the same step.
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
// a few hundred bytes per (n, h).  One workgroup per (n, h) with up to 1024 threads:
// thread (rg, cg) holds rows rg, rg+RG, ... of the 4 state columns cg*4..cg*4+3 in
// registers, so the state never leaves registers between its load and its store, and
// each thread has only a few 16-byte loads in flight (a wide workgroup with short
// per-thread streams keeps more of HBM busy than a narrow one with long streams).
// The column sums p, r are reduced within each wave by shuffles, across waves
// through LDS by one thread per (column group, component), which also forms u and o.
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

template <int DK, int DV> struct DecodeMap {
    static constexpr int CG = DV / 4;                                  // float4 column groups
    static constexpr int RG = (DK < 1024 / CG) ? DK : 1024 / CG;       // row groups
    static constexpr int RPT = DK / RG;                                // rows per thread
    static constexpr int NT = CG * RG;                                 // threads
    static constexpr int NTB = NT < WAVE ? WAVE : NT;                  // block (whole waves)
    static constexpr int NWV = NTB / WAVE;
};

// MODE 0 (DECODE_STEP): one token per sequence, o written, state updated in place.
// MODE 1 (DECODE_VERIFY): n_tok draft tokens per sequence, o written for each, the state
//   kept in registers only: the caller's state is left as it was, since an in-place update
//   could not be rolled back after a rejected draft.
// MODE 2 (DECODE_COMMIT): the state advanced by the first n_accept[n] draft tokens of
//   sequence n, replayed from their cached per-token inputs (q, k, v, gate, beta: far
//   smaller than the state), no o.
// Both follow orkas.ai "Kimi K3 architecture", section "The cost comes back in the serving
// stack" (speculative decoding).  Token j of sequence n, head h sits at token-head index
// (n n_tok + j) H + h of q, k, v, the gates, beta and o.
// NORM: q and k are L2-normalised per token inside the kernel.  It is a compile-time
// choice because its reductions, even untaken, push the plain step past the 64 VGPRs
// that 8 waves per SIMD allow and make it spill.
template <typename ET, int DK, int DV, int MODE, bool NORM>
__global__ __launch_bounds__((DecodeMap<DK, DV>::NTB)) __attribute__((amdgpu_waves_per_eu(8))) void decode_kernel(
    float* __restrict__ state, const ET* __restrict__ q, const ET* __restrict__ k,
    const ET* __restrict__ v, const float* __restrict__ log_alpha,
    const float* __restrict__ beta, ET* __restrict__ o, const int* __restrict__ n_accept,
    int H, int n_tok, unsigned flags) {
    using DM = DecodeMap<DK, DV>;
    constexpr int CG = DM::CG, RG = DM::RG, RPT = DM::RPT, NT = DM::NT, NWV = DM::NWV;
    static_assert(DK % RG == 0 && DK <= NT && 4 * CG <= NT, "decode thread map");
    constexpr bool want_o = MODE != DECODE_COMMIT;
    constexpr bool write_state = MODE != DECODE_VERIFY;

    const size_t unit = blockIdx.x;                 // n H + h
    const size_t n = unit / (unsigned)H, h = unit - n * (unsigned)H;
    const int tid = threadIdx.x;
    const bool act = tid < NT;                      // (small shapes: the last wave is partial)
    const int cg = tid % CG, rg = tid / CG;
    const int w = tid / WAVE;

    // per-token vectors (decay factors, k, q), double-buffered by token parity: token j+1
    // writes its copy while threads may still read token j's in the state update
    __shared__ float s_tok[2][3][DK];
    __shared__ f32x4 s_p[NWV][CG], s_r[NWV][CG];
    __shared__ float s_kq[NWV], s_kk[NWV], s_qq[NWV];   // per-wave k.q, |k|^2, |q|^2
    __shared__ f32x4 s_u[CG];
    const int gate = flags & FLAG_GATE_LOGITS;
    constexpr bool norm = NORM;                     // q, k normalised per token

    f32x4* S = reinterpret_cast<f32x4*>(state + unit * (size_t)(DK * DV));
    f32x4 sv[RPT];
    if (act) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) sv[i] = __builtin_nontemporal_load(&S[(rg + i * RG) * CG + cg]);
    }
    int cnt = MODE == DECODE_STEP ? 1 : n_tok;
    if (MODE == DECODE_COMMIT) cnt = min(max(n_accept[n], 0), n_tok);

    // Per-token inputs are loaded one token ahead, in their storage types (converted where
    // they are used), so their memory latency overlaps the previous token's reductions:
    // gate, k, q for lanes tid < DK; v (column tid) and beta for the reducer lanes tid < DV.
    // Addresses are a uniform per-token base plus a 32-bit lane offset; beta goes through a
    // lane-varying (zero) offset so that it is a vector load like the rest, not a scalar
    // load that would be waited for on the spot.
    const unsigned ut = (unsigned)tid;
    unsigned zero = 0;
    asm volatile("" : "+v"(zero));
    float la_n = 0.f, b_n = 0.f;
    ET k_n{}, q_n{}, v_n{};
    auto load_tok = [&](int j) {
        const size_t th = (n * (unsigned)n_tok + j) * (unsigned)H + h;   // token-head index
        if (tid < DK) {
            la_n = (log_alpha + th * DK)[ut];
            k_n = (k + th * DK)[ut];
            if (want_o) q_n = (q + th * DK)[ut];
        }
        if (tid < DV) {
            v_n = (v + th * DV)[ut];
            b_n = (beta + th)[zero];
        }
    };
    if (cnt > 0) load_tok(0);

    for (int j = 0; j < cnt; ++j) {
        const int buf = j & 1;
        const float la_c = la_n, b_c = b_n;
        const ET k_c = k_n, q_c = q_n, v_c = v_n;
        if (j + 1 < cnt) load_tok(j + 1);
        float* s_a = s_tok[buf][0];
        float* s_k = s_tok[buf][1];
        float* s_q = s_tok[buf][2];
        // With normalisation the raw k and q go to LDS and their norms scale the results
        // instead: p and u by 1/|k|, r by 1/|q|, k.q by both (the reducer applies them).
        float kq = 0.f, k2 = 0.f, q2 = 0.f;
        if (tid < DK) {
            const float kk = to_f32(k_c);
            s_a[tid] = fast_exp(log_decay(la_c, gate));
            s_k[tid] = kk;
            k2 = kk * kk;
            if (want_o) {
                const float qq = to_f32(q_c);
                s_q[tid] = qq;
                kq = kk * qq;
                q2 = qq * qq;
            }
        }
        if (want_o) {
#pragma unroll
            for (int m = WAVE / 2; m >= 1; m >>= 1) kq += __shfl_xor(kq, m);
            if ((tid & (WAVE - 1)) == 0) s_kq[w] = kq;
        }
        if (norm) {
#pragma unroll
            for (int m = WAVE / 2; m >= 1; m >>= 1) {
                k2 += __shfl_xor(k2, m);
                if (want_o) q2 += __shfl_xor(q2, m);
            }
            if ((tid & (WAVE - 1)) == 0) {
                s_kk[w] = k2;
                s_qq[w] = q2;
            }
        }
        __syncthreads();

        // decay the state; partial column sums p = (DS)^T k, r = (DS)^T q over this thread's rows
        f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
        if (act) {
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int row = rg + i * RG;
                sv[i] *= s_a[row];
                p += sv[i] * s_k[row];
                if (want_o) r += sv[i] * s_q[row];
            }
        }
        // reduce over the row groups that share a wave (lanes differing in bits >= log2 CG)
#pragma unroll
        for (int m = CG; m < WAVE; m <<= 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                p[e] += __shfl_xor(p[e], m);
                if (want_o) r[e] += __shfl_xor(r[e], m);
            }
        }
        if ((tid & (WAVE - 1)) < CG) {
            s_p[w][cg] = p;
            if (want_o) s_r[w][cg] = r;
        }
        __syncthreads();

        // one thread per (column group, component) = column tid: u = beta (v - p), o = r + (k . q) u
        if (tid < DV) {
            const int rc = tid >> 2, re = tid & 3;
            float P = 0.f, R = 0.f, KQ = 0.f;
#pragma unroll
            for (int ww = 0; ww < NWV; ++ww) {
                P += s_p[ww][rc][re];
                if (want_o) {
                    R += s_r[ww][rc][re];
                    KQ += s_kq[ww];
                }
            }
            float ik = 1.f, iq = 1.f;                   // 1 / |k|, 1 / |q| (normalisation)
            if (norm) {
                float KK = 0.f, QQ = 0.f;
#pragma unroll
                for (int ww = 0; ww < NWV; ++ww) {
                    KK += s_kk[ww];
                    QQ += s_qq[ww];
                }
                ik = __builtin_amdgcn_rsqf(KK + QK_NORM_EPS);
                iq = __builtin_amdgcn_rsqf(QQ + QK_NORM_EPS);
            }
            const float u = b_c * (to_f32(v_c) - P * ik);
            s_u[rc][re] = u * ik;                       // the update adds raw k times u / |k|
            if (want_o) {
                const size_t th = (n * (unsigned)n_tok + j) * (unsigned)H + h;
                (o + th * DV)[ut] = from_f32<ET>(R * iq + KQ * ik * iq * u);
            }
        }
        __syncthreads();

        if (act) {
            const f32x4 u = s_u[cg];
#pragma unroll
            for (int i = 0; i < RPT; ++i) sv[i] += s_k[rg + i * RG] * u;
        }
    }
    if (write_state && act) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) __builtin_nontemporal_store(sv[i], &S[(rg + i * RG) * CG + cg]);
    }
}

template <typename ET, int DK, int DV, int MODE>
static hipError_t launch_decode_m(const DecodeArgs& a, hipStream_t st) {
    const unsigned nblk = (unsigned)(a.N * a.H);
    if (a.flags & FLAG_QK_L2NORM)
        hipLaunchKernelGGL((decode_kernel<ET, DK, DV, MODE, true>), dim3(nblk), dim3(DecodeMap<DK, DV>::NTB), 0,
                           st, a.state, (const ET*)a.q, (const ET*)a.k, (const ET*)a.v, a.log_alpha, a.beta,
                           (ET*)a.o, a.n_accept, (int)a.H, (int)a.n_tok, a.flags);
    else
        hipLaunchKernelGGL((decode_kernel<ET, DK, DV, MODE, false>), dim3(nblk), dim3(DecodeMap<DK, DV>::NTB), 0,
                           st, a.state, (const ET*)a.q, (const ET*)a.k, (const ET*)a.v, a.log_alpha, a.beta,
                           (ET*)a.o, a.n_accept, (int)a.H, (int)a.n_tok, a.flags);
    return hipGetLastError();
}

template <typename ET, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
    switch (a.mode) {
        case DECODE_STEP: return launch_decode_m<ET, DK, DV, DECODE_STEP>(a, st);
        case DECODE_VERIFY: return launch_decode_m<ET, DK, DV, DECODE_VERIFY>(a, st);
        case DECODE_COMMIT: return launch_decode_m<ET, DK, DV, DECODE_COMMIT>(a, st);
    }
    return hipErrorInvalidValue;
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
