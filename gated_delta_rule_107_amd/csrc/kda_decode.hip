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

template <int DK, int DV, int MAXT = 1024> struct DecodeMap {
    static constexpr int CG = DV / 4;                                  // float4 column groups
    static constexpr int RG = (DK < MAXT / CG) ? DK : MAXT / CG;       // row groups
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
// that 8 waves per SIMD allow and make it spill; the normalising instantiations run at
// 4 waves per SIMD instead (up to 128 VGPRs, 76-85 used at 128 x 128), where they do not
// spill (at 8 they spilled up to 72 bytes per thread and were 1-2 % slower).
template <typename ET, int DK, int DV, int MODE, bool NORM>
__global__ __launch_bounds__((DecodeMap<DK, DV>::NTB)) __attribute__((amdgpu_waves_per_eu(NORM ? 4 : 8))) void decode_kernel(
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

// positions of A_ts (s < t) and M_ts (s <= t) among a group's small products
__host__ __device__ constexpr int a_index(int t, int s) { return t * (t - 1) / 2 + s; }
__host__ __device__ constexpr int m_index(int t, int s) { return 6 + t * (t + 1) / 2 + s; }

// Speculative verify in chunk form.  Verify never writes the state, so instead of n
// successive steps (three barriers each) it evaluates its drafts in groups of up to VG as one
// chunk from the state in registers, with Gamma_t the cumulative log-decay over the group's
// drafts 0..t:
//     X_t = S^T (k_t e^Gamma_t),  Y_t = S^T (q_t e^Gamma_t)                 (one pass over S)
//     A_ts = sum_c k_tc k_sc e^(Gamma_tc - Gamma_sc)  (s < t),  M_ts = ... q_tc ...  (s <= t)
//     u_t = beta_t (v_t - X_t - sum_{s<t} A_ts u_s),  o_t = Y_t + sum_{s<=t} M_ts u_s
// which is the token recurrence unrolled over the group (the chunk equations at chunk length
// VG).  A group costs two barriers: after the per-draft vectors and small products, and after
// the partial column sums.  Longer draft lists advance the register state between groups,
// S <- Diag(e^Gamma_last) S + sum_t (k_t e^(Gamma_last - Gamma_t)) u_t^T, so no cumulative
// decay spans more than VG drafts.  With normalisation the raw k, q are used and the norms
// scale the results in the reducer.
// 256 threads per (n, h), 16 state rows each, at up to 168 VGPRs (3 waves per SIMD): three
// workgroups, i.e. three states, per CU in flight (at 512 threads and 8 rows two fitted, and
// verify was 8 % slower; at 4 waves per SIMD the 256-thread form spills).  A group's
// per-draft inputs are loaded before the state (the first group) or during the previous
// group, so that neither the small products nor the solve wait for memory.
constexpr int VERIFY_THREADS = 256;
template <typename ET, int DK, int DV, bool NORM>
__global__ __launch_bounds__((DecodeMap<DK, DV, VERIFY_THREADS>::NTB)) __attribute__((amdgpu_waves_per_eu(3))) void verify_kernel(
    const float* __restrict__ state, const ET* __restrict__ q, const ET* __restrict__ k,
    const ET* __restrict__ v, const float* __restrict__ log_alpha, const float* __restrict__ beta,
    ET* __restrict__ o, int H, int n_tok, unsigned flags) {
    using DM = DecodeMap<DK, DV, VERIFY_THREADS>;
    constexpr int CG = DM::CG, RG = DM::RG, RPT = DM::RPT, NT = DM::NT, NWV = DM::NWV;
    constexpr int VG = 4;                                // drafts per group
    constexpr int NA = VG * (VG - 1) / 2, NM = VG * (VG + 1) / 2;
    constexpr int NSM = NA + NM + 2 * VG;                // small products per channel
    static_assert(m_index(0, 0) == NA, "small-product positions assume groups of 4");
    constexpr int NCW = (DK + WAVE - 1) / WAVE;          // waves of the channel threads
    static_assert(DK % RG == 0 && DK <= NT && 4 * CG <= NT && DV <= NT, "verify thread map");
    static_assert(NSM <= WAVE, "one lane per small product sums its row partials");

    const size_t unit = blockIdx.x;                      // n H + h
    const size_t n = unit / (unsigned)H, h = unit - n * (unsigned)H;
    const int tid = threadIdx.x;
    const bool act = tid < NT;
    const int cg = tid % CG, rg = tid / CG;
    const int w = tid / WAVE, lane = tid & (WAVE - 1);
    const int gate = flags & FLAG_GATE_LOGITS;

    __shared__ float s_kt[VG][DK], s_qt[VG][DK], s_kh[VG][DK], s_eg[DK];
    __shared__ float s_sm[NCW * 4][NSM];                 // per 16-lane row sums of the small products
    __shared__ float s_smt[NSM];                         // the small products
    __shared__ f32x4 s_xy[NWV][2 * VG][CG];              // per-wave partial column sums of X_t, Y_t
    __shared__ float s_u[VG][DV];                        // the group's u (scaled by 1/|k|), between groups

    // A group's inputs in their storage types: gate, k, q of channel tid (tid < DK) and v of
    // column tid, beta (tid < DV).  Token-head addresses are a uniform base plus a 32-bit lane
    // offset; beta goes through a lane-varying zero offset so that it is a vector load.
    const unsigned ut = (unsigned)tid;
    unsigned zero = 0;
    asm volatile("" : "+v"(zero));
    float la_g[VG], b_g[VG];
    ET k_g[VG], q_g[VG], v_g[VG];
    auto load_group = [&](int j0) {
#pragma unroll
        for (int t = 0; t < VG; ++t) {
            const bool in = j0 + t < n_tok;
            const size_t th = (n * (unsigned)n_tok + (in ? j0 + t : 0)) * (unsigned)H + h;
            if (tid < DK && in) {
                la_g[t] = (log_alpha + th * DK)[ut];
                k_g[t] = (k + th * DK)[ut];
                q_g[t] = (q + th * DK)[ut];
            }
            if (tid < DV && in) {
                v_g[t] = (v + th * DV)[ut];
                b_g[t] = (beta + th)[zero];
            }
        }
    };
    load_group(0);

    const f32x4* S = reinterpret_cast<const f32x4*>(state + unit * (size_t)(DK * DV));
    f32x4 sv[RPT];
    if (act) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) sv[i] = __builtin_nontemporal_load(&S[(rg + i * RG) * CG + cg]);
    }

    for (int j0 = 0; j0 < n_tok; j0 += VG) {
        const int ng = n_tok - j0 < VG ? n_tok - j0 : VG;
        const bool more = j0 + VG < n_tok;
        if (j0 > 0) __syncthreads();                     // the previous group's readers are done
        // ---- (1) per-draft vectors of channel c = tid, and the small products
        if (w < NCW) {
            const int c = tid;
            const bool on = c < DK;
            float kk[VG], qq[VG], gm[VG], gam = 0.f;
#pragma unroll
            for (int t = 0; t < VG; ++t) {
                kk[t] = qq[t] = 0.f;
                if (on && t < ng) {
                    gam += log_decay(la_g[t], gate);
                    kk[t] = to_f32(k_g[t]);
                    qq[t] = to_f32(q_g[t]);
                }
                gm[t] = gam;
            }
            float sm[NSM];
#pragma unroll
            for (int t = 0; t < VG; ++t) {
#pragma unroll
                for (int s2 = 0; s2 <= t; ++s2) {
                    const float d = fast_exp(gm[t] - gm[s2]);          // <= 1
                    if (s2 < t) sm[a_index(t, s2)] = kk[t] * kk[s2] * d;
                    sm[m_index(t, s2)] = qq[t] * kk[s2] * d;
                }
                sm[NA + NM + t] = kk[t] * kk[t];
                sm[NA + NM + VG + t] = qq[t] * qq[t];
            }
            if (on) {
                const float egl = fast_exp(gm[VG - 1]);
#pragma unroll
                for (int t = 0; t < VG; ++t) {
                    const float e = fast_exp(gm[t]);
                    s_kt[t][c] = kk[t] * e;
                    s_qt[t][c] = qq[t] * e;
                    s_kh[t][c] = kk[t] * (egl / e);
                }
                s_eg[c] = egl;
            }
            // sums over each 16-lane row (DPP row shifts); the row's last lane holds the sum
#pragma unroll
            for (int i = 0; i < NSM; ++i) {
                float x = sm[i];
                x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xF, 0xF, true));
                x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xF, 0xF, true));
                x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xF, 0xF, true));
                x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xF, 0xF, true));
                if ((lane & 15) == 15) s_sm[w * 4 + (lane >> 4)][i] = x;
            }
        }
        __syncthreads();

        // ---- (2) partial column sums of X_t = S^T kt_t and Y_t = S^T qt_t over this thread's
        // rows; lanes of the last wave also sum the small products' row partials
        if (act) {
#pragma unroll
            for (int t = 0; t < VG; ++t) {
                if (t >= ng) break;
                f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < RPT; ++i) {
                    const int row = rg + i * RG;
                    x += sv[i] * s_kt[t][row];
                    y += sv[i] * s_qt[t][row];
                }
#pragma unroll
                for (int m = CG; m < WAVE; m <<= 1) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[e] += __shfl_xor(x[e], m);
                        y[e] += __shfl_xor(y[e], m);
                    }
                }
                if (lane < CG) {
                    s_xy[w][2 * t][cg] = x;
                    s_xy[w][2 * t + 1][cg] = y;
                }
            }
        }
        if (w == NWV - 1 && lane < NSM) {
            float x = 0.f;
#pragma unroll
            for (int r = 0; r < NCW * 4; ++r) x += s_sm[r][lane];
            s_smt[lane] = x;
        }
        // the next group's gates, k and q (read in (1) above, before the barrier)
        if (more && tid < DK) {
#pragma unroll
            for (int t = 0; t < VG; ++t) {
                const int j = j0 + VG + t;
                if (j < n_tok) {
                    const size_t th = (n * (unsigned)n_tok + j) * (unsigned)H + h;
                    la_g[t] = (log_alpha + th * DK)[ut];
                    k_g[t] = (k + th * DK)[ut];
                    q_g[t] = (q + th * DK)[ut];
                }
            }
        }
        __syncthreads();

        // ---- (3) one thread per value column: the group's solve and outputs
        if (tid < DV) {
            const int rc = tid >> 2, re = tid & 3;
            float ik[VG], iq[VG];
#pragma unroll
            for (int t = 0; t < VG; ++t) {
                ik[t] = NORM ? __builtin_amdgcn_rsqf(s_smt[NA + NM + t] + QK_NORM_EPS) : 1.f;
                iq[t] = NORM ? __builtin_amdgcn_rsqf(s_smt[NA + NM + VG + t] + QK_NORM_EPS) : 1.f;
            }
            float u[VG];
#pragma unroll
            for (int t = 0; t < VG; ++t) {
                u[t] = 0.f;
                if (t < ng) {
                    float X = 0.f, Y = 0.f;
#pragma unroll
                    for (int ww = 0; ww < NWV; ++ww) {
                        X += s_xy[ww][2 * t][rc][re];
                        Y += s_xy[ww][2 * t + 1][rc][re];
                    }
                    float acc = to_f32(v_g[t]) - X * ik[t];
#pragma unroll
                    for (int s2 = 0; s2 < t; ++s2) acc -= s_smt[a_index(t, s2)] * ik[t] * ik[s2] * u[s2];
                    u[t] = b_g[t] * acc;
                    float ot = Y * iq[t];
#pragma unroll
                    for (int s2 = 0; s2 <= t; ++s2) ot += s_smt[m_index(t, s2)] * iq[t] * ik[s2] * u[s2];
                    const size_t th = (n * (unsigned)n_tok + j0 + t) * (unsigned)H + h;
                    (o + th * DV)[ut] = from_f32<ET>(ot);
                }
            }
            if (more) {
#pragma unroll
                for (int t = 0; t < VG; ++t) s_u[t][tid] = u[t] * ik[t];   // the update adds raw k
            }
        }
        if (more) {
            // the next group's v and beta
            if (tid < DV) {
#pragma unroll
                for (int t = 0; t < VG; ++t) {
                    const int j = j0 + VG + t;
                    if (j < n_tok) {
                        const size_t th = (n * (unsigned)n_tok + j) * (unsigned)H + h;
                        v_g[t] = (v + th * DV)[ut];
                        b_g[t] = (beta + th)[zero];
                    }
                }
            }
            __syncthreads();
            // ---- (4) advance the register state over the group
            if (act) {
#pragma unroll
                for (int i = 0; i < RPT; ++i) {
                    const int row = rg + i * RG;
                    sv[i] *= s_eg[row];
#pragma unroll
                    for (int t = 0; t < VG; ++t) {
                        const f32x4 ut4 = *reinterpret_cast<const f32x4*>(&s_u[t][4 * cg]);
                        sv[i] += s_kh[t][row] * ut4;
                    }
                }
            }
        }
    }
}

template <typename ET, int DK, int DV>
static hipError_t launch_verify(const DecodeArgs& a, hipStream_t st) {
    const unsigned nblk = (unsigned)(a.N * a.H);
    if (a.flags & FLAG_QK_L2NORM)
        hipLaunchKernelGGL((verify_kernel<ET, DK, DV, true>), dim3(nblk), dim3(DecodeMap<DK, DV, VERIFY_THREADS>::NTB), 0, st,
                           a.state, (const ET*)a.q, (const ET*)a.k, (const ET*)a.v, a.log_alpha, a.beta, (ET*)a.o,
                           (int)a.H, (int)a.n_tok, a.flags);
    else
        hipLaunchKernelGGL((verify_kernel<ET, DK, DV, false>), dim3(nblk), dim3(DecodeMap<DK, DV, VERIFY_THREADS>::NTB), 0, st,
                           a.state, (const ET*)a.q, (const ET*)a.k, (const ET*)a.v, a.log_alpha, a.beta, (ET*)a.o,
                           (int)a.H, (int)a.n_tok, a.flags);
    return hipGetLastError();
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
        case DECODE_VERIFY: return launch_verify<ET, DK, DV>(a, st);
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
