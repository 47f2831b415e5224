// Chunked KDA prefill for gfx950: the work of one workgroup, shared by the chunk kernel
// (kda_chunk.hip) and the lead kernel of segmented plans (kda_chunk_lead.hip).
//
// Each workgroup owns one (batch, head, segment, column block) and walks its
// chunks of C tokens in order.  Per chunk, with Gamma the inclusive cumulative
// sum of the floored log-decay g from the chunk start and S the start state:
//
//   A[t,s] = sum_c k_tc k_sc e^(Gamma_tc - Gamma_sc)   (s <  t)
//   M[t,s] = sum_c q_tc k_sc e^(Gamma_tc - Gamma_sc)   (s <= t)
//   U  = (I + Diag(beta) A)^-1 Diag(beta) (V - (k e^Gamma) S)          (WY/UT form)
//   O  = (q e^Gamma) S + M U
//   S' = Diag(e^Gamma_C) S + (k e^(Gamma_C - Gamma))^T U
//
// Chunked evaluation has to divide by a cumulative decay; the floor on the
// log-decay bounds a 16-token tile's cumulative log-decay to [-80, 0], so its
// reciprocal stays below e^80 ~ 5.5e34, inside bf16, and the diagonal tiles
// run as the same dense matrix products as every other tile (orkas.ai "Kimi
// K3 architecture", section "The floor that removed a GPU code path").
//
// Reference points.  Let t lie in 16-token sub-tile p of the chunk, gamma_t
// the inclusive cumulative log-decay inside that sub-tile, tot_p its total,
// r_p = tot_0 + ... + tot_{p-1}, so Gamma_t = r_p + gamma_t.  Stored operands:
//   KL = k e^gamma, QL = q e^gamma, RH = k e^(tot_p - gamma)       (all <= 1)
//   Kt = KL e^(r_p) = k e^Gamma, Qt = q e^Gamma                    (<= 1, may flush to 0)
//   KhT = (k e^(Gamma_C - Gamma))^T                                (<= 1)
// A and M tiles are (KL or QL) Diag(f) RH^T with f = e^-tot_p (<= e^80, the
// diagonal tile), f = 1 for adjacent sub-tiles and f = e^(r_p - r_pp+1) (<= 1)
// further below.  bf16 operands fold f into right-operand variants that gate prep
// stores (RD = RH e^-tot_p; RF = RH e^tot_{pp+1}, RH e^(tot_{pp+1} + tot_{pp+2})); float32
// operands apply f to the left operand in registers.
//
// Per chunk: gate prep from registers prefetched a chunk ahead writes the operands
// above to LDS; A / M tiles run on MFMA together with X = Kt S, QS = Qt S; the four
// 16x16 diagonal blocks of (I + Diag(beta) A) are inverted by fp32 forward
// substitution; then the state chain runs per wave on its 16 state columns: the
// block triangular solve for U on MFMA straight from registers
// (U_p = N_pp (R_p - sum_q Ab_pq U_q)), O, and the state update.  In the solve N_pp,
// Ab_pq = -beta A_pq and U are bf16 operands, but R_p enters the N_pp product split into
// bf16 high and low parts: rounding R_p alone carried nearly all of the solve's rounding
// error into U and the state.  The loop is
// software-pipelined by one chunk: the chain of chunk n (MFMA latency) shares its
// barrier interval with the gate prep of chunk n+1 (VALU work).  The fp32 state
// stays in MFMA accumulators for the whole sequence; accumulator tiles feed the next
// product's B operand directly (the contraction index is taken in the order the
// accumulator layout holds it, and the LDS operand is read in that same order).
//
// bf16 inputs use v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x16_bf16 with
// fp32 accumulation; float32 inputs use v_mfma_f32_16x16x4_f32 throughout.
#pragma once

#include "kda_chunk_ops.h"
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

// ---------------------------------------------------------------- one workgroup's work
// `bid` is the workgroup's index in its launch's grid (the chunk kernel passes blockIdx.x; the
// lead kernel its index within the part of the grid that runs this MODE).
// MODE 0: outputs and final states; MODE 1: segment summaries (see ChunkArgs).
// EXT: the optional features of a call (state checkpoints in MODE 0, gate logits, q / k
// normalisation), switched by the arguments at run time.  A separate instantiation: their
// code, even never taken, costs the plain loop several per cent.
template <typename OpT, int DK, int C, int MODE, bool EXT>
__device__ __forceinline__ void chunk_body(const ChunkArgs& a, const int64_t bid) {
    constexpr bool CK = EXT && MODE == 0;             // checkpoints: one-pass / pass-2 kernel only
    using MF = MM<OpT>;
    using B16 = typename MF::B16;
    using L4 = Ld4<OpT>;
    using V4 = typename L4::V;
    constexpr int E = sizeof(OpT);
    constexpr bool RV = E == 2;
    constexpr int PADE = 16 / E;
    constexpr int NT = C / 16;                       // 16-token sub-tiles per chunk
    constexpr int NCT = DK / 16;                     // 16-row tiles of the state
    constexpr int DKP = DK < 32 ? 32 : DK;
    // Row pitches (LDS has 32 4-byte banks; 16 lanes of a b64 access and 8 lanes of a b128
    // access share a cycle).  Tiles read 16 B per lane (the natural-order A / M operands):
    // pitch = 4 banks mod 32, so 8 consecutive rows hit 8 distinct bank quads.  Tiles read
    // 8 B per lane (the chained operands Kt, Qt, Khat^T, the solve and M blocks): pitch = 2
    // banks mod 32, so 16 consecutive rows hit 16 distinct bank pairs.  (bf16; float32 keeps
    // 16-byte pitches so its 16-byte chained loads stay aligned.)  Other pitches measured
    // slower: Kt / Qt at DKP + 8 by 10 %, the C-wide tiles at C + 8 by 3 %.
    constexpr int LDK = DKP + PADE;
    constexpr int LKQ = DKP + 4;
    constexpr int LC = C + 4;
    constexpr int KNAT = (E == 2) ? (DK + 31) / 32 : DK / 4;   // natural-order steps over channels
    constexpr bool want_o = MODE == 0;
    // state column groups per wave: one in MODE 0; in MODE 1 the widened state [S | M] as two,
    // 16 value columns (S, from 0, values v) and 16 transition columns (M, from I, values 0)
    constexpr int NG = MODE == 1 ? 2 : 1;
    constexpr Lds L = lds_layout(E, DK, C);

    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    OpT* s_kt = reinterpret_cast<OpT*>(smem + L.kt);
    OpT* s_qt = reinterpret_cast<OpT*>(smem + L.qt);
    OpT* s_kl = reinterpret_cast<OpT*>(smem + L.kl);
    OpT* s_ql = reinterpret_cast<OpT*>(smem + L.ql);
    OpT* s_rh = reinterpret_cast<OpT*>(smem + L.rh);
    OpT* s_rd = reinterpret_cast<OpT*>(smem + L.rd);
    OpT* s_rf = reinterpret_cast<OpT*>(smem + L.rf);
    OpT* s_kht = reinterpret_cast<OpT*>(smem + L.kht);
    OpT* s_an = reinterpret_cast<OpT*>(smem + L.an);
    OpT* s_mm = reinterpret_cast<OpT*>(smem + L.mm);
    float* s_ad = reinterpret_cast<float*>(smem + L.ad);    // [p][s][t]: transposed diagonal blocks
    float* s_fd = reinterpret_cast<float*>(smem + L.fd);
    float* s_fo = reinterpret_cast<float*>(smem + L.fo);
    float* s_egc = reinterpret_cast<float*>(smem + L.egc);
    float* s_beta = reinterpret_cast<float*>(smem + L.beta);

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    __builtin_assume(wave >= 0 && wave < 8);

    // ---- which (batch, head, segment, column block) this workgroup owns.  Column blocks of
    // one unit are 8 block indices apart, so they share an XCD (blocks go round-robin over 8).
    // MODE 1 has one block: every wave holds both of its column groups.
    const int H = a.H, dv = a.dv;
    const int DVB = MODE == 0 ? a.dv_block : dv;    // value columns of this workgroup
    const int ncb = MODE == 0 ? dv / DVB : 1;
    // this launch covers segments seg_lo .. seg_lo + seg_cnt - 1 (pass 1 of packed sequences covers
    // every slot and skips the last segments itself)
    const int nseg_grid = a.seg_cnt;
    int64_t unit, cb;
    {
        const int64_t grp = bid / (8 * ncb), rem = bid % (8 * ncb);
        unit = grp * 8 + rem % 8;
        cb = rem / 8;
        const int64_t nunits = a.B * H * (int64_t)nseg_grid;
        const int64_t tail0 = (nunits / 8) * 8;            // last, partial group of 8 units
        if (grp * 8 >= tail0) {
            const int64_t ntail = nunits - tail0, r2 = bid - tail0 * ncb;
            unit = tail0 + r2 % ntail;
            cb = r2 / ntail;
        }
    }
    const int seg = a.seg_lo + (int)(unit % nseg_grid);
    const int64_t bh = unit / nseg_grid;                 // (sequence, head): indexes pairs and starts
    const int h = (int)(bh % H);
    const int64_t T = a.T;
    int64_t b = bh / H, t_begin, t_end;                 // b, t: index the token tensors
    int64_t srow = bh;                                   // state row of S0 / S_T: (sequence, head)
    bool last_seg = seg == a.n_seg - 1;
    if (a.seg_table) {
        // packed sequences with segments: this slot's sequence and token range (the whole
        // workgroup returns together, before any barrier, for an empty slot, and in pass 1
        // for a sequence's last segment)
        const int4 e = a.seg_table[seg];
        if (e.x < 0 || (MODE == 1 && (e.w & SEG_LAST))) return;
        b = 0;
        srow = (int64_t)e.x * H + h;
        t_begin = e.y;
        t_end = e.z;
        last_seg = (e.w & SEG_LAST) != 0;
    } else if (a.cu_seqlens) {
        // packed sequences (one pass): sequence bh / H owns tokens [cu[i], cu[i+1]) of the
        // single batch row; offsets are clamped into [0, T], so bad offsets cannot fault
        const int64_t i = b;
        b = 0;
        const int64_t c0 = a.cu_seqlens[i], c1 = a.cu_seqlens[i + 1];
        t_begin = c0 < 0 ? 0 : (c0 > T ? T : c0);
        t_end = c1 < t_begin ? t_begin : (c1 > T ? T : c1);
    } else {
        // segment 0 has its own length in the lead form (seg0_len > 0), the others seg_len
        const int64_t len0 = a.seg0_len > 0 ? a.seg0_len : a.seg_len;
        const int64_t len = seg == 0 ? len0 : a.seg_len;
        t_begin = seg == 0 ? 0 : len0 + (int64_t)(seg - 1) * a.seg_len;
        t_end = t_begin + len < T ? t_begin + len : T;
    }

    const int colw = (int)cb * DVB + 16 * wave;      // first value column of this wave
    const bool chain = 16 * wave < DVB;              // this wave owns value columns
    const bool mchain = MODE == 1 && 16 * wave < DK; // ... transition columns 16w.. of M (MODE 1)
    // Where this unit's final state goes, fixed here so that one pointer, not its ingredients,
    // stays live across the chunk loop: MODE 0 the last segment's S_T, or in the lead form
    // segment 0's final state (the true start of segment 1); MODE 1 the pair's slots.
    float* fin_s = nullptr;
    bf16* fin_m = nullptr;
    if constexpr (MODE == 0) {
        if (last_seg) fin_s = a.s_final + srow * DK * dv;
        else if (a.seg0_len > 0 && seg == 0 && !a.seg_table) fin_s = a.starts + (bh * a.n_seg + 1) * DK * dv;
    } else {
        fin_s = a.s_loc + (bh * a.n_seg + seg) * DK * dv;
        fin_m = reinterpret_cast<bf16*>(a.m_tr) + (bh * a.n_seg + seg) * 2 * DK * DK;
    }

    const OpT* gq = reinterpret_cast<const OpT*>(a.q);
    const OpT* gk = reinterpret_cast<const OpT*>(a.k);
    const OpT* gv = reinterpret_cast<const OpT*>(a.v);
    OpT* go = reinterpret_cast<OpT*>(a.o);
    const int tok_k = H * DK;                        // elements between tokens in q, k, log_alpha
    const int tok_v = H * dv;                        // ... in v and o

    // ---- zero LDS once (gate prep clears the padding channels of DK < 32 with every chunk)
    for (int i = threadIdx.x * 16; i < L.total; i += 512 * 16)
        *reinterpret_cast<f32x4*>(smem + i) = f32x4{0.f, 0.f, 0.f, 0.f};

    // Thread maps.  Gate prep: wave w holds channels 16w..16w+15; lane = 16 p + 4 i + x
    // covers the channel quad c0 = 16w + 4x and the token quad tq = 4p + i (tokens
    // 4tq..4tq+3 of sub-tile p), so a 16-lane DPP row is one sub-tile and a 16-lane store
    // pass spans 4 token quads x 4 channel quads.
    // Chain: wave w holds state columns colw..colw+15; lane (g, jl) holds rows 4g..4g+3 of
    // each 16-row tile in column jl (the accumulator layout), and v / o in that layout.
    // Lane-derived indices are recomputed from an opaque copy of the thread id inside the
    // chunk loop, so the compiler does not hoist dozens of per-lane addresses out of the
    // loop and hold them in registers for its whole length.

    // prefetch registers (one chunk ahead)
    f32x4 pla[4];
    V4 pk[4], pq[4];
    // v granules of 16 bytes: thread tid holds granules tid, tid + 512, ... of the chunk's
    // [C][DVB] value block (row = granule / GPR, granule column = granule % GPR)
    typedef __attribute__((__vector_size__(16))) float g16;
    constexpr int NGV = C * (128 * E / 16) / 512 > 0 ? C * (128 * E / 16) / 512 : 1;
    g16 pv[NGV];
    float pbeta = 0.f;

    // Loads are unconditional, from addresses clamped into the tensors: tokens past the end
    // are masked where they are used, one chunk later, so no instruction here waits for the
    // data.  beta is loaded under exactly the predicate of its consumer, so no path reaches
    // the next prefetch with that load unconsumed.
    // Row offsets use 24-bit multiplies (the ABI bounds H * max(dk, dv) below 2^24).  When the
    // whole chunk is in range, token j of each quad is one stride further: an add, no clamp.
    // The lane map covers 64 tokens; with C < 64 the lanes of sub-tiles C/16.. are idle and
    // their token quad is clamped to the chunk's last one (their values are never used, and
    // on a sequence's last chunk they would otherwise read past the end of the tensors).
    auto prefetch_gates = [&](int64_t t0, int tid) {
        const int lane = tid & 63;
        const int tq = min(4 * (lane >> 4) + ((lane >> 2) & 3), C / 4 - 1);
        const int gc0 = min(16 * wave + 4 * (lane & 3), DK - 4);
        const int tlim = (int)(t_end - 1 - t0 < C - 1 ? t_end - 1 - t0 : C - 1);
        const int64_t base = ((b * T + t0) * H + h) * (int64_t)DK;       // uniform
        const float* la_b = a.log_alpha + base;
        const OpT* k_b = gk + base;
        const OpT* q_b = gq + base;
        if (tlim == C - 1) {
            unsigned off = tok_elem_off(4 * tq, tok_k, gc0);
#pragma unroll
            for (int j = 0; j < 4; ++j, off += tok_k) {
                pla[j] = *at_bytes(reinterpret_cast<const f32x4*>(la_b), off * 4u);
                pk[j] = *at_bytes(reinterpret_cast<const V4*>(k_b), off * (unsigned)E);
                if (want_o) pq[j] = *at_bytes(reinterpret_cast<const V4*>(q_b), off * (unsigned)E);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const unsigned off = tok_elem_off(min(4 * tq + j, tlim), tok_k, gc0);
                pla[j] = *at_bytes(reinterpret_cast<const f32x4*>(la_b), off * 4u);
                pk[j] = *at_bytes(reinterpret_cast<const V4*>(k_b), off * (unsigned)E);
                if (want_o) pq[j] = *at_bytes(reinterpret_cast<const V4*>(q_b), off * (unsigned)E);
            }
        }
        if (tid < C) pbeta = *at_bytes(a.beta + (b * T + t0) * H + h, tok_elem_off(min(tid, tlim), H, 0) * 4u);
    };
    // v for the chain as 16-byte granules (GPR per row); rows past the end read a clamped row
    // and are multiplied by beta = 0 later, transition columns are zeroed when staged
    constexpr int VG = 16 / E;                       // elements per granule
    const int GPR = DVB / VG;                        // granules per row of the value block
    // granule index -> (row, granule column) without a division per use: multiply by the
    // rounded-up reciprocal 2^32 / GPR and keep the high word (exact for indices < 2^16)
    const unsigned gpr_magic = 0xFFFFFFFFu / (unsigned)GPR + 1u;
    auto granule = [&](int gi2, int& row, int& gc) {
        row = (int)__umulhi((unsigned)gi2, gpr_magic);
        gc = gi2 - row * GPR;
    };
    auto prefetch_v = [&](int64_t t0, int tid) {
        const int tlim = (int)(t_end - 1 - t0 < C - 1 ? t_end - 1 - t0 : C - 1);
        const OpT* v_b = gv + ((b * T + t0) * H + h) * (int64_t)dv + (int)cb * DVB;   // uniform
#pragma unroll
        for (int u = 0; u < NGV; ++u) {
            const int gi2 = tid + 512 * u;
            int row, gc;
            granule(gi2, row, gc);
            const int col = min(gc * VG, dv - (int)cb * DVB - VG);
            if (row < C) pv[u] = *at_bytes(reinterpret_cast<const g16*>(v_b), tok_elem_off(min(row, tlim), tok_v, col) * (unsigned)E);
        }
    };
    // staging tile for the next chunk's v, over the Kt..RF region, which is dead between the
    // A / M tiles and the next gate prep
    constexpr int LVO = 128 + PADE;                  // pitch: up to 128 columns
    OpT* s_v = s_kt;
    static_assert(C * LVO * E <= L.kht - L.kt, "v staging tile exceeds the dead operand region");

    // ---- start state into accumulator layout: Sacc[G][tau][r] = S[16 tau + g4 + r][colw + jl]
    // (group 1: M[16 tau + g4 + r][16 w + jl], from the identity)
    f32x4 Sacc[NG][NCT];
    {
        const int lane = threadIdx.x & 63, g4 = 4 * (lane >> 4), jl = lane & 15;
        const float* src = nullptr;
        if (MODE == 0) {
            // with segments every start comes from the scan's output (segment 0's included), so
            // S0 is never read here while another workgroup writes S_T; in the lead form segment 0
            // starts from S0 in a launch that writes no S_T
            if (!a.seg_table && (a.n_seg == 1 || (a.seg0_len > 0 && seg == 0)))
                src = a.s0 ? a.s0 + bh * DK * dv : nullptr;
            else src = a.starts + (bh * a.n_seg + seg) * DK * dv;
        }
#pragma unroll
        for (int tau = 0; tau < NCT; ++tau)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * tau + g4 + r;
                Sacc[0][tau][r] = (chain && src) ? src[row * dv + colw + jl] : 0.f;
                if constexpr (NG == 2) Sacc[1][tau][r] = (mchain && row == 16 * wave + jl) ? 1.f : 0.f;
            }
    }

    // Optional q / k normalisation.  For the chunk whose k and q sit in the prefetch
    // registers, each wave sums the squares of its 16 channels per token; the partials go to
    // the diagonal-block area of LDS (dead from phase 4 until the next phase 2) as
    // [wave][token][k, q], and gate prep scales k and q by 1 / sqrt(sum + eps) before use.
    const bool qk_norm = EXT && (a.flags & FLAG_QK_L2NORM);
    float* s_nrm = s_ad;
    static_assert(8 * C * 2 * 4 <= NT * 16 * 16 * 4, "normalisation partials exceed their LDS area");
    auto norm_partials = [&](int tid) {
        const int lane = tid & 63;
        const int tq = 4 * (lane >> 4) + ((lane >> 2) & 3);        // this lane's prefetched token quad
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float kf[4], qf[4], kk = 0.f, qq = 0.f;
            L4::to_f(pk[j], kf);
#pragma unroll
            for (int e = 0; e < 4; ++e) kk += kf[e] * kf[e];
            if (want_o) {
                L4::to_f(pq[j], qf);
#pragma unroll
                for (int e = 0; e < 4; ++e) qq += qf[e] * qf[e];
            }
            kk += quad_xor<1>(kk);                               // the wave's 4 channel quads
            kk += quad_xor<2>(kk);
            qq += quad_xor<1>(qq);
            qq += quad_xor<2>(qq);
            if ((lane & 3) == 0 && tq < C / 4) {
                s_nrm[(wave * C + 4 * tq + j) * 2] = kk;
                s_nrm[(wave * C + 4 * tq + j) * 2 + 1] = qq;
            }
        }
    };

    __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0): the start state is in registers
    const int64_t nchunks = t_end > t_begin ? (t_end - t_begin + C - 1) / C : 0;
    if (nchunks > 0) {
        prefetch_gates(t_begin, threadIdx.x);
        prefetch_v(t_begin, threadIdx.x);
        if constexpr (EXT) {
            if (qk_norm) {
                __syncthreads();                     // LDS zeroing done before the partials land
                norm_partials(threadIdx.x);
            }
        }
    }

    // Software pipeline over chunks.  Iteration n runs the state chain of chunk n and prepares
    // chunk n+1; its four barriers separate
    //   (1) chain(n) [R, U, O, S update]  +  gate prep(n+1)    (MFMA latency next to VALU work)
    //   (2) Khat^T(n+1) to LDS, X / QS(n+1) from the updated state, A / M tiles(n+1)
    //   (3) diagonal-block inverses(n+1), v(n+1) into its staging tile
    //   (4) v(n+1) into registers in the accumulator layout.
    // beta and e^Gamma_C of chunk n are read in (1) while gate prep writes chunk n+1's, so
    // they have two slots (chunk n uses slot n & 1); Khat^T(n+1) waits in registers until (2).
    f32x4 X[NG][NT], QS[NT];                         // Kt S, (Qt S)^T of the chunk chained next
    B16 vr[NT];                                      // its v (value columns)
    V4 khr[4];                                       // Khat^T(n+1): 4 channels x 4 tokens

    // state checkpoints (pass 2 / one pass): tokens into this unit's range that end the next
    // one (-1: none), and where it goes (this head's columns of checkpoint t / stride - 1)
    int ck_rel = -1;
    float* ck_ptr = nullptr;
    if (CK && a.ckpt) {
        const int64_t first = t_begin / a.ckpt_stride;            // index of the next checkpoint
        ck_rel = (int)((first + 1) * a.ckpt_stride - t_begin);
        ck_ptr = a.ckpt + ((b * (T / a.ckpt_stride) + first) * H + h) * (int64_t)DK * dv + colw;
    }

    auto body = [&](auto cur_c, auto nxt_c, int64_t n) {
        constexpr bool cur = decltype(cur_c)::value;  // a chain runs (chunk n exists)
        constexpr bool nxt = decltype(nxt_c)::value;  // chunk n+1 exists
        const int64_t t0 = t_begin + n * C, t1 = t0 + C;
        const int Tc = cur ? (int)(t_end - t0 < C ? t_end - t0 : C) : 0;
        const int Tn = nxt ? (int)(t_end - t1 < C ? t_end - t1 : C) : 0;
        float* sb_c = s_beta + (int)(n & 1) * C;
        float* eg_c = s_egc + (int)(n & 1) * DKP;
        float* sb_n = s_beta + (int)((n + 1) & 1) * C;
        float* eg_n = s_egc + (int)((n + 1) & 1) * DKP;
        int tid_opaque = threadIdx.x;
        asm volatile("" : "+v"(tid_opaque));
        const int tid = tid_opaque, lane = tid & 63;
        const int g4 = 4 * (lane >> 4), jl = lane & 15;
        const int gx = lane & 3, gi = (lane >> 2) & 3, gp = lane >> 4;
        const int tq = 4 * gp + gi;
        const int gc0 = 16 * wave + 4 * gx;
        const bool gact = gc0 < DK && gp < NT;
        __syncthreads();   // the previous iteration's readers of the staging tiles are done
        // Branches stay at phase boundaries: the chain and the gate prep below form one block
        // in which the compiler interleaves MFMA and VALU work.
        if constexpr (nxt && EXT) {
            if (a.flags & FLAG_GATE_LOGITS) {        // raw logits: log-decay -5 sigmoid (uniform)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) pla[j][e] = gate_from_logit(pla[j][e]);
            }
            if (qk_norm) {                           // k, q of chunk n+1 scaled to unit norm (uniform)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int t = min(4 * tq + j, C - 1);           // (idle lanes: any token)
                    float sk = 0.f, sq = 0.f;
#pragma unroll
                    for (int w2 = 0; w2 < NCT; ++w2) {
                        sk += s_nrm[(w2 * C + t) * 2];
                        sq += s_nrm[(w2 * C + t) * 2 + 1];
                    }
                    const float ik = __builtin_amdgcn_rsqf(sk + QK_NORM_EPS);
                    float f[4];
                    L4::to_f(pk[j], f);
#pragma unroll
                    for (int e = 0; e < 4; ++e) f[e] *= ik;
                    pk[j] = L4::from_f(f);
                    if (want_o) {
                        const float iq = __builtin_amdgcn_rsqf(sq + QK_NORM_EPS);
                        L4::to_f(pq[j], f);
#pragma unroll
                        for (int e = 0; e < 4; ++e) f[e] *= iq;
                        pq[j] = L4::from_f(f);
                    }
                }
            }
        }

        // ================= (1a) chain of chunk n: R_p = beta (V - X); U_p = N_pp (R_p - sum_{q<p} Ab_pq U_q)
        // (the transition columns of MODE 1 have V = 0)
        B16 ub[NG][NT];
        if constexpr (cur) {
#pragma unroll
            for (int p = 0; p < NT; ++p) {
                f32x4 R[NG];
#pragma unroll
                for (int G = 0; G < NG; ++G)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        R[G][r] = sb_c[16 * p + g4 + r] * ((G == 0 ? (float)vr[p][r] : 0.f) - X[G][p][r]);
                // each solve tile is loaded once for every column group
#pragma unroll
                for (int q = 0; q < p; ++q) {
                    const typename MF::A16 an = MF::ld16(s_an, LC, 16 * p, 16 * q, lane);
#pragma unroll
                    for (int G = 0; G < NG; ++G) R[G] = MF::mma16(an, ub[G][q], R[G]);
                }
                const typename MF::A16 nd = MF::ld16(s_an, LC, 16 * p, 16 * p, lane);
#pragma unroll
                for (int G = 0; G < NG; ++G) ub[G][p] = MF::b16(MF::mma16_split(nd, R[G]));
            }
        }

        // ================= (1c) O = QS + M U of chunk n, stored straight from the accumulators
        // (its store instructions issue while the gate prep below keeps the vector units busy).
        // QS and O are held transposed: lane (g, jl) holds token 16 p + jl, value columns 4g ..
        // 4g+3, written by one store; rows past the chunk's last token (and every row of a wave
        // without value columns) fall outside the store's buffer range and are dropped.  The
        // range, Tc token rows, stays below 64 * 2^24 * 4 bytes = 2^32 by the bound on H * dv.
        if constexpr (cur && want_o) {
            const unsigned rowb = (unsigned)tok_v * E;
            const __amdgpu_buffer_rsrc_t o_rs =
                bounded_rsrc(go + ((b * T + t0) * H + h) * (int64_t)dv + colw, chain ? (unsigned)Tc * rowb : 0u);
            const unsigned o_off = tok_elem_off(jl, tok_v, g4) * (unsigned)E;
#pragma unroll
            for (int p = 0; p < NT; ++p) {
#pragma unroll
                for (int qq = 0; qq <= p; ++qq) QS[p] = MF::k16t(s_mm, LC, 16 * p, 16 * qq, ub[0][qq], QS[p], lane);
                Store4<OpT>::st(o_rs, o_off + 16 * p * rowb, QS[p]);
            }
        }

        // ================= (1b) gate prep of chunk n+1 (log-decays in log2 units from here on)
        float g2[4][4];
        float pre[4], tot[4], rp[4], after[4], gcs[4], tn1[4], tn2[4], tm1[4], tm2[4];
        const bool full = !(NT < 4 || Tn < C);
        if constexpr (nxt) {
            if (tid < C) sb_n[tid] = tid < Tn ? pbeta : 0.f;
            // Every lane runs the cross-lane scans; only stores are guarded.  Tokens past the
            // end (and lanes past the last sub-tile) read clamped addresses: their log-decay is
            // zeroed here (idle channel lanes of DK < 128 only feed their own 16-lane rows,
            // whose stores are skipped).  k and q stay in their packed prefetch registers until
            // they are used.
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // tokens past the end scale by 0 (their loads read a clamped, valid token)
                const float sc = (full || 4 * tq + j < Tn) ? LOG2E : 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) g2[j][e] = clamp_log_alpha(pla[j][e]) * sc;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float loc = g2[0][e] + g2[1][e] + g2[2][e] + g2[3][e];
                // inclusive scan over the 4 token quads of this sub-tile (lanes 4 apart)
                float inc = loc;
                inc += row_shr<4>(inc);
                inc += row_shr<8>(inc);
                pre[e] = row_shr<4>(inc);                             // exclusive
                // sub-tile totals from lane 12 + x of every row
                float tp[4];
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) tp[qq] = qq < NT ? __shfl(inc, 16 * qq + 12 + gx, 64) : 0.f;
                tot[e] = gp == 0 ? tp[0] : gp == 1 ? tp[1] : gp == 2 ? tp[2] : tp[3];
                rp[e] = (gp > 0 ? tp[0] : 0.f) + (gp > 1 ? tp[1] : 0.f) + (gp > 2 ? tp[2] : 0.f);  // r_p
                gcs[e] = tp[0] + tp[1] + tp[2] + tp[3];               // Gamma_C
                after[e] = gcs[e] - rp[e] - tot[e];                   // later sub-tiles
                tn1[e] = gp == 0 ? tp[1] : gp == 1 ? tp[2] : gp == 2 ? tp[3] : 0.f;   // sub-tile p+1
                tn2[e] = gp == 0 ? tp[2] : gp == 1 ? tp[3] : 0.f;                      // p+2
                tm1[e] = gp == 1 ? tp[0] : gp == 2 ? tp[1] : gp == 3 ? tp[2] : 0.f;   // p-1
                tm2[e] = gp == 2 ? tp[0] : gp == 3 ? tp[1] : 0.f;                      // p-2
            }
        }

        // ================= (1d) gate prep of chunk n+1: operands to LDS
        if constexpr (nxt) {
            if (gact && gi == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (gp == 0) eg_n[gc0 + e] = fast_exp2(gcs[e]);
                    if (!RV) {
                        s_fd[gp * DKP + gc0 + e] = fast_exp2(-tot[e]);                               // e^-tot_p
                        if (NT == 4 && gp == 2) s_fo[0 * DKP + gc0 + e] = fast_exp2(tm1[e]);          // (2,0)
                        if (NT == 4 && gp == 3) {
                            s_fo[1 * DKP + gc0 + e] = fast_exp2(tm1[e] + tm2[e]);                     // (3,0)
                            s_fo[2 * DKP + gc0 + e] = fast_exp2(tm1[e]);                              // (3,1)
                        }
                    }
                }
            }
            if (gact) {
                const unsigned okq0 = (unsigned)(4 * tq * LKQ + gc0) * E, okl0 = (unsigned)(4 * tq * LDK + gc0) * E;
                float er[4], eh[4], ed[4], ef1[4], ef2[4], gam[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    er[e] = fast_exp2(rp[e]);
                    eh[e] = fast_exp2(after[e]);
                    gam[e] = pre[e];
                    if (RV) {
                        ed[e] = fast_exp2(-tot[e]);
                        ef1[e] = fast_exp2(tn1[e]);
                        ef2[e] = fast_exp2(tn1[e] + tn2[e]);
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // tokens past the end keep their (clamped, finite) k and q: their beta is 0
                    // and their log-decay 0, so they change neither U, O nor the state
                    float k[4][4], q[4][4];
                    L4::to_f(pk[j], k[j]);
                    if (want_o) L4::to_f(pq[j], q[j]);
                    else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) q[j][e] = 0.f;
                    }
                    float kl[4], ql[4], rh[4], kt[4], qt[4], rd[4], rf1[4], rf2[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        gam[e] += g2[j][e];
                        const float e1 = fast_exp2(gam[e]), e2 = fast_exp2(tot[e] - gam[e]);
                        kl[e] = k[j][e] * e1;
                        ql[e] = q[j][e] * e1;
                        rh[e] = k[j][e] * e2;
                        kt[e] = kl[e] * er[e];
                        qt[e] = ql[e] * er[e];
                        khr[e][j] = from_f32<OpT>(rh[e] * eh[e]);    // Khat^T: [channel][token]
                        if (RV) {
                            rd[e] = rh[e] * ed[e];                    // k e^-gamma, <= e^80
                            rf1[e] = rh[e] * ef1[e];                  // referenced at the end of p+1
                            rf2[e] = rh[e] * ef2[e];                  // ... of p+2
                        }
                    }
                    // byte offsets: a per-lane part computed once plus constants (token j of the
                    // quad, the array's place in LDS), which the stores take as immediates
                    const unsigned okq = okq0 + j * (LKQ * E), okl = okl0 + j * (LDK * E);
                    *at_bytes(reinterpret_cast<V4*>(s_kt), okq) = L4::from_f(kt);
                    *at_bytes(reinterpret_cast<V4*>(s_kl), okl) = L4::from_f(kl);
                    *at_bytes(reinterpret_cast<V4*>(s_rh), okl) = L4::from_f(rh);
                    if (want_o) {
                        *at_bytes(reinterpret_cast<V4*>(s_qt), okq) = L4::from_f(qt);
                        *at_bytes(reinterpret_cast<V4*>(s_ql), okl) = L4::from_f(ql);
                    }
                    if (RV) {
                        *at_bytes(reinterpret_cast<V4*>(s_rd), okl) = L4::from_f(rd);
                        if (NT == 4 && gp <= 1) *at_bytes(reinterpret_cast<V4*>(s_rf), okl) = L4::from_f(rf1);
                        if (NT == 4 && gp == 0) *at_bytes(reinterpret_cast<V4*>(s_rf), okl + 32 * LDK * E) = L4::from_f(rf2);
                    }
                }
            }
        }

        if constexpr (nxt && DK < DKP) {
            // channels DK..DKP-1 pad the 32-deep natural-order products; the staging tiles
            // overwrite them, so they are cleared with every chunk's operands
            if (gc0 >= DK && gc0 < DKP && gp < NT) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int t = 4 * tq + j;
                    const V4 z = L4::zero();
                    *reinterpret_cast<V4*>(s_kl + t * LDK + gc0) = z;
                    *reinterpret_cast<V4*>(s_ql + t * LDK + gc0) = z;
                    *reinterpret_cast<V4*>(s_rh + t * LDK + gc0) = z;
                    if (RV) {
                        *reinterpret_cast<V4*>(s_rd + t * LDK + gc0) = z;
                        if (NT == 4 && gp <= 1) *reinterpret_cast<V4*>(s_rf + t * LDK + gc0) = z;
                        if (NT == 4 && gp == 0) *reinterpret_cast<V4*>(s_rf + (32 + t) * LDK + gc0) = z;
                    }
                }
            }
        }

        // ================= (1e) S <- Diag(e^Gamma_C) S + Khat^T U for chunk n (every column
        // group from one load of each Khat^T tile)
        if constexpr (cur) {
#pragma unroll
            for (int tau = 0; tau < NCT; ++tau) {
                const f32x4 eg = *reinterpret_cast<const f32x4*>(eg_c + 16 * tau + g4);
#pragma unroll
                for (int G = 0; G < NG; ++G)
#pragma unroll
                    for (int r = 0; r < 4; ++r) Sacc[G][tau][r] *= eg[r];
                if constexpr (NT == 1) {
#pragma unroll
                    for (int G = 0; G < NG; ++G)
                        Sacc[G][tau] = MF::k16(s_kht, LC, 16 * tau, 0, ub[G][0], Sacc[G][tau], lane);
                } else {
#pragma unroll
                    for (int s2 = 0; s2 < NT / 2; ++s2) {
                        const typename MF::A32 kh = MF::ld32(s_kht, LC, 16 * tau, 32 * s2, lane);
#pragma unroll
                        for (int G = 0; G < NG; ++G)
                            Sacc[G][tau] = MF::mma32(kh, ub[G][2 * s2], ub[G][2 * s2 + 1], Sacc[G][tau]);
                    }
                }
            }
        }
        // chunk n+2's gates, keys and queries load while chunk n+1 is processed
        if (nxt && n + 2 < nchunks) prefetch_gates(t1 + C, tid);
        __syncthreads();

        // state checkpoint after tokens [0, t0 + C) when that is a multiple of the stride
        // (Sacc holds the state after chunk n)
        if constexpr (cur && CK) {
            if ((int)(n + 1) * C == ck_rel) {        // (never true without checkpoints)
                if (chain && t_begin + ck_rel <= T) {
#pragma unroll
                    for (int tau = 0; tau < NCT; ++tau)
#pragma unroll
                        for (int r = 0; r < 4; ++r) ck_ptr[(16 * tau + g4 + r) * dv + jl] = Sacc[0][tau][r];
                }
                ck_rel += (int)a.ckpt_stride;
                ck_ptr += (int64_t)H * DK * dv;
            }
        }

        // ================= (2) Khat^T(n+1) to LDS; X = Kt S and QS = Qt S; the A / M tiles
        if constexpr (nxt) {
            if (gact) {
#pragma unroll
                for (int e = 0; e < 4; ++e) *reinterpret_cast<V4*>(s_kht + (gc0 + e) * LC + 4 * tq) = khr[e];
            }
            {
                B16 sb[NG][NCT];
#pragma unroll
                for (int G = 0; G < NG; ++G)
#pragma unroll
                    for (int tau = 0; tau < NCT; ++tau) sb[G][tau] = MF::b16(Sacc[G][tau]);
                if constexpr (NCT == 1 || E == 4) {
                    // (float32 operands are 4x larger: no room to hold a second sub-tile's)
#pragma unroll
                    for (int p = 0; p < NT; ++p) {
#pragma unroll
                        for (int G = 0; G < NG; ++G) X[G][p] = f32x4{0.f, 0.f, 0.f, 0.f};
                        QS[p] = f32x4{0.f, 0.f, 0.f, 0.f};
                        if constexpr (NCT == 1) {
#pragma unroll
                            for (int G = 0; G < NG; ++G) X[G][p] = MF::k16(s_kt, LKQ, 16 * p, 0, sb[G][0], X[G][p], lane);
                            if (want_o) QS[p] = MF::k16t(s_qt, LKQ, 16 * p, 0, sb[0][0], QS[p], lane);
                        } else {
#pragma unroll
                            for (int s2 = 0; s2 < NCT / 2; ++s2) {
#pragma unroll
                                for (int G = 0; G < NG; ++G)
                                    X[G][p] = MF::k32(s_kt, LKQ, 16 * p, 32 * s2, sb[G][2 * s2], sb[G][2 * s2 + 1],
                                                      X[G][p], lane);
                                if (want_o)
                                    QS[p] = MF::k32t(s_qt, LKQ, 16 * p, 32 * s2, sb[0][2 * s2], sb[0][2 * s2 + 1], QS[p],
                                                     lane);
                            }
                        }
                    }
                } else {
                    // Software-pipelined over the sub-tiles: the operand loads of sub-tile p+1
                    // are issued before the products of sub-tile p (scheduling barriers keep the
                    // compiler from pulling them back next to their uses).
                    typename MF::A32 ax[2][NCT / 2], aq[2][NCT / 2];
                    auto load = [&](int p, int buf) {
#pragma unroll
                        for (int s2 = 0; s2 < NCT / 2; ++s2) {
                            ax[buf][s2] = MF::ld32(s_kt, LKQ, 16 * p, 32 * s2, lane);
                            if (want_o) aq[buf][s2] = MF::ld32(s_qt, LKQ, 16 * p, 32 * s2, lane);
                        }
                    };
                    load(0, 0);
#pragma unroll
                    for (int p = 0; p < NT; ++p) {
                        if (p + 1 < NT) load(p + 1, (p + 1) & 1);
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int G = 0; G < NG; ++G) X[G][p] = f32x4{0.f, 0.f, 0.f, 0.f};
                        QS[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s2 = 0; s2 < NCT / 2; ++s2) {
#pragma unroll
                            for (int G = 0; G < NG; ++G)
                                X[G][p] = MF::mma32(ax[p & 1][s2], sb[G][2 * s2], sb[G][2 * s2 + 1], X[G][p]);
                            if (want_o) QS[p] = MF::mma32t(aq[p & 1][s2], sb[0][2 * s2], sb[0][2 * s2 + 1], QS[p]);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
            // Tile tasks: sub-tile pairs (p, pp <= p), row by row.  With outputs, a task computes
            // the A tile and the M tile of its pair, which share the right operand (read once);
            // every task's loads and products come before any of the wave's stores.
            constexpr int NPAIR = NT * (NT + 1) / 2;
            constexpr int NSLOT = (NPAIR + 7) / 8;
            // With outputs and more than 8 pairs (64-token chunks: 10), the pairs past the first 8
            // are split into their A and M tiles, one tile per wave (waves 0 .. 2 (NPAIR - 8) - 1),
            // so that no wave carries two pairs; a split tile reads its right operand itself.
            constexpr bool SPLIT = want_o && NPAIR > 8;
            static_assert(!SPLIT || (NSLOT == 2 && 2 * (NPAIR - 8) <= 8), "tile split assumes one extra slot");
            auto pair_of = [&](int task, int& p, int& pp) {
                int pr = task;
                p = 0;
                while (pr > p) { pr -= p + 1; ++p; }
                pp = pr;                                          // pp <= p
            };
            auto right_of = [&](int p, int pp, const OpT*& right, int& rrow, const float*& fac) {
                right = s_rh;
                rrow = 16 * pp;
                fac = nullptr;
                if (RV) {
                    if (p == pp) right = s_rd;
                    else if (p - pp == 2) right = s_rf;                           // rows 16 pp
                    else if (p - pp == 3) { right = s_rf; rrow = 32 + 16 * pp; }
                } else {
                    fac = p == pp ? s_fd + p * DKP : (p - pp >= 2 ? s_fo + pair_fo_index(p, pp) * DKP : nullptr);
                }
            };
            f32x4 acc[NSLOT], accm[NSLOT];
#pragma unroll
            for (int sl = 0; sl < NSLOT; ++sl) {
                acc[sl] = f32x4{0.f, 0.f, 0.f, 0.f};
                accm[sl] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (SPLIT && sl == 1) {
                    if (wave < 2 * (NPAIR - 8)) {                 // tile (wave & 1 ? M : A) of pair 8 + wave / 2
                        int p, pp, rrow;
                        pair_of(8 + wave / 2, p, pp);
                        const OpT* right;
                        const float* fac;
                        right_of(p, pp, right, rrow, fac);
                        const OpT* left = (wave & 1) ? s_ql : s_kl;
#pragma unroll
                        for (int ks = 0; ks < KNAT; ++ks)
                            acc[sl] = MF::nat(left, LDK, 16 * p, right, LDK, rrow, ks * MF::KS, fac, acc[sl], lane);
                    }
                    continue;
                }
                const int task = wave + 8 * sl;
                if (task < NPAIR) {
                    int p, pp, rrow;
                    pair_of(task, p, pp);
                    const OpT* right;
                    const float* fac;
                    right_of(p, pp, right, rrow, fac);
#pragma unroll
                    for (int ks = 0; ks < KNAT; ++ks) {
                        if constexpr (want_o)
                            MF::nat2(s_kl, s_ql, LDK, 16 * p, right, LDK, rrow, ks * MF::KS, fac, acc[sl], accm[sl], lane);
                        else
                            acc[sl] = MF::nat(s_kl, LDK, 16 * p, right, LDK, rrow, ks * MF::KS, fac, acc[sl], lane);
                    }
                }
            }
            // an A tile: the diagonal block of beta A goes to s_ad (strictly lower, transposed:
            // [p][s][t]), the others, as -beta A, to s_an; an M tile goes to s_mm (masked on the diagonal)
            auto store_a = [&](int p, int pp, const f32x4& x) {
                if (p == pp) {
                    f32x4 col;
#pragma unroll
                    for (int r = 0; r < 4; ++r) col[r] = (jl < g4 + r) ? x[r] * sb_n[16 * p + g4 + r] : 0.f;
                    *reinterpret_cast<f32x4*>(s_ad + (p * 16 + jl) * 16 + g4) = col;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 16 * p + g4 + r, s = 16 * pp + jl;
                        s_an[t * LC + s] = from_f32<OpT>(-x[r] * sb_n[t]);
                    }
                }
            };
            auto store_m = [&](int p, int pp, const f32x4& x) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tr = g4 + r;
                    const int t = 16 * p + tr, s = 16 * pp + jl;
                    s_mm[t * LC + s] = from_f32<OpT>((p == pp && jl > tr) ? 0.f : x[r]);
                }
            };
#pragma unroll
            for (int sl = 0; sl < NSLOT; ++sl) {
                if (SPLIT && sl == 1) {
                    if (wave < 2 * (NPAIR - 8)) {
                        int p, pp;
                        pair_of(8 + wave / 2, p, pp);
                        if (wave & 1) store_m(p, pp, acc[sl]);
                        else store_a(p, pp, acc[sl]);
                    }
                    continue;
                }
                const int task = wave + 8 * sl;
                if (task < NPAIR) {
                    int p, pp;
                    pair_of(task, p, pp);
                    store_a(p, pp, acc[sl]);
                    if constexpr (want_o) store_m(p, pp, accm[sl]);
                }
            }
        }
        __syncthreads();

        // ================= (3) inverses of the diagonal blocks of I + Diag(beta) A (fp32), by
        // forward substitution on the identity: wave p inverts block p with its rows across the
        // lanes (lane 16 r + t holds row t of columns 4r .. 4r+3), so a step is four FMAs whose
        // x_s comes from lane s of the same 16-lane row
        if constexpr (nxt) {
            if (wave < NT) {
                const int p = wave, t = lane & 15, r4 = 4 * (lane >> 4);
                const float* Ab = s_ad + p * 256;                // column s at Ab[16 s .. 16 s + 15]
                float nl[15], x[4];
#pragma unroll
                for (int s = 0; s < 15; ++s) nl[s] = -Ab[16 * s + t];        // -beta A[t][s], 0 unless s < t
#pragma unroll
                for (int c = 0; c < 4; ++c) x[c] = (t == r4 + c) ? 1.f : 0.f;
                rows_forward_subst(x, nl);
                *reinterpret_cast<V4*>(s_an + (16 * p + t) * LC + 16 * p + r4) = L4::from_f(x);
            }
            // v(n+1) into its staging tile (transition columns of pass 1 read zeros)
#pragma unroll
            for (int u = 0; u < NGV; ++u) {
                const int gi2 = tid + 512 * u;
                int row, gc;
                granule(gi2, row, gc);
                if (row < C) *reinterpret_cast<g16*>(s_v + row * LVO + gc * VG) = pv[u];
            }
            if (n + 2 < nchunks) prefetch_v(t1 + C, tid);
        }
        __syncthreads();

        // ================= (4) v(n+1) into the accumulator layout; normalisation partials of
        // chunk n+2, whose k and q the prefetch registers now hold
        if constexpr (nxt) {
#pragma unroll
            for (int p = 0; p < NT; ++p)
#pragma unroll
                for (int r = 0; r < 4; ++r) vr[p][r] = s_v[(16 * p + g4 + r) * LVO + 16 * wave + jl];
            if constexpr (EXT) {
                if (qk_norm && n + 2 < nchunks) norm_partials(tid);
            }
        }
    };

    if (nchunks > 0) {
        body(BoolC<false>{}, BoolC<true>{}, -1);
        if constexpr (EXT) {
            // (the loop entered only when it runs: in this instantiation the compiler otherwise
            // spills values that skip the loop around it)
            if (nchunks > 1) {
                int64_t n = 0;
                do body(BoolC<true>{}, BoolC<true>{}, n);
                while (++n + 1 < nchunks);
            }
        } else {
            for (int64_t n = 0; n + 1 < nchunks; ++n) body(BoolC<true>{}, BoolC<true>{}, n);
        }
        body(BoolC<true>{}, BoolC<false>{}, nchunks - 1);
    }

    // ---- final state of this unit
    {
        const int lane = threadIdx.x & 63, g4 = 4 * (lane >> 4), jl = lane & 15;
        const int col = colw + jl;
        if constexpr (MODE == 0) {
            if (chain && fin_s) {
#pragma unroll
                for (int tau = 0; tau < NCT; ++tau)
#pragma unroll
                    for (int r = 0; r < 4; ++r) fin_s[(16 * tau + g4 + r) * dv + col] = Sacc[0][tau][r];
            }
        } else {
            if (chain) {
                // the zero-start state goes to the scan in its accumulator-tile order
                float* sl = fin_s;
#pragma unroll
                for (int tau = 0; tau < NCT; ++tau)
                    *reinterpret_cast<f32x4*>(sl + sloc_index(DK, 16 * tau + g4, col)) = Sacc[0][tau];
            }
            if (mchain) {
                // the transition goes to the scan already split into bf16 high and low planes, in
                // the order of the scan's A operand
                bf16* mh = fin_m;
#pragma unroll
                for (int tau = 0; tau < NCT; ++tau)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float x = Sacc[NG - 1][tau][r];
                        const bf16 hi = (bf16)x;
                        const int at = mtr_index(DK, 16 * tau + g4 + r, 16 * wave + jl);
                        mh[at] = hi;
                        mh[DK * DK + at] = (bf16)(x - (float)hi);
                    }
            }
        }
    }
}

}  // namespace kda
