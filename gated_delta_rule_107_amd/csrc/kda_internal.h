// Host-side launch interface between the C ABI layer (kda_api.cpp) and the
// HIP kernels.  Arguments are validated by the ABI layer before they get here.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// kda_input_flag_t bits as the kernels see them
constexpr uint32_t FLAG_GATE_LOGITS = 1u, FLAG_QK_L2NORM = 2u;
constexpr float QK_NORM_EPS = 1e-6f;          // x / sqrt(sum x^2 + eps)

// Decode modes: one step (state updated in place); verify n_tok draft tokens (outputs only,
// the state read but not written); commit the first n_accept[n] of n_tok tokens (state only).
enum { DECODE_STEP = 0, DECODE_VERIFY = 1, DECODE_COMMIT = 2 };

struct DecodeArgs {
    float* state;
    const void *q, *k, *v;
    const float *log_alpha, *beta;   // log_alpha: log-decays or raw logits (gate)
    void* o;                         // null for commit
    const int32_t* n_accept;         // [N] (commit), else null
    int64_t N;
    int32_t n_tok;                   // tokens per sequence (1 for a step)
    int32_t H, dk, dv;
    int32_t mode;
    uint32_t flags;                  // kda_input_flag_t bits (gate logits, q/k L2 normalisation)
    bool bf16;
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);

// One launch of the chunk kernel covers every (batch, head, segment, column block).
//   mode 0: full evaluation of each segment from its start state; writes o and,
//           for the last segment, the final state.
//   mode 1: segment summaries (pass 1) for segments 0 .. n_seg-2: the state is
//           widened to [S | M] (dv + dk columns) started from [0 | I] with value
//           columns [v | 0]; writes S_loc (dk x dv) and M (dk x dk) per segment.
struct ChunkArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta;
    const float* s0;        // [B,H,dk,dv] or null (zeros): start state when n_seg == 1 (mode 0)
    float* starts;          // [B,H,P,dk,dv] start state of every segment (read by mode 0 when
                            // n_seg > 1; the lead form's segment 0 writes the start of segment 1)
    void* o;                // [B,T,H,dv] (mode 0)
    float* s_final;         // [B,H,dk,dv] (mode 0)
    float* s_loc;           // [B,H,P][dk dv] (mode 1), each block in sloc_index order
    void* m_tr;             // [B,H,P][2][dk^2] bf16 (mode 1): M split into high and low parts,
                            // each plane in the scan's operand order (mtr_index)
    int64_t B, T;           // with cu_seqlens: B = number of sequences, T = packed tokens
    int32_t H, dk, dv, chunk;
    int32_t n_seg;          // P
    int64_t seg_len;        // tokens per segment, a multiple of chunk
    int64_t seg0_len;       // tokens of segment 0 in the lead form (then segment i > 0 starts at
                            // seg0_len + (i - 1) seg_len), 0 = every segment seg_len long
    int32_t seg_lo, seg_cnt;  // this launch covers segments seg_lo .. seg_lo + seg_cnt - 1
    int32_t dv_block;       // columns per workgroup (16 per wave)
    const int32_t* cu_seqlens;  // [B + 1] packed sequence offsets into one batch row, or null
    // packed sequences with segments (seg_table non-null; B = 1, n_seg = the table's length):
    // entry g = {sequence or -1, t_begin, t_end, SEG_FIRST | SEG_LAST}; state rows are
    // sequences, and pairs / start states of slot g of head h sit at index h * n_seg + g
    const int4* seg_table;
    float* ckpt;            // [B, T / ckpt_stride, H, dk, dv] state checkpoints (mode 0) or null
    int64_t ckpt_stride;    // tokens between checkpoints, a multiple of chunk
    uint32_t flags;         // kda_input_flag_t bits (gate logits, q/k L2 normalisation)
    int32_t mode;
    bool bf16;
};

hipError_t launch_chunk(const ChunkArgs& a, hipStream_t st);

// Lead form of a segmented plan, one launch: a0 (mode 0) runs segment 0 of every (batch, head,
// column block) from S0 and writes its final state to starts[.., 1]; a1 (mode 1) runs pass 1 over
// segments 1 .. P-2.  a1.seg_cnt may be 0.
hipError_t launch_chunk_lead(const ChunkArgs& a0, const ChunkArgs& a1, hipStream_t st);

// Prefix scan over segment pairs: starts[i+1] = M_i starts[i] + S_loc_i.  first = 0: starts[0]
// = s0 (or zeros), writes starts[0 .. P-1]; first = 1 (lead form): starts[1] is given, writes
// starts[2 .. P-1] from pairs 1 .. P-2.
struct ScanArgs {
    const float* s0;
    const float* s_loc;     // [B,H,P][dk dv], sloc_index order
    const void* m_tr;       // [B,H,P][2][dk^2] bf16: high and low parts of M (hi + lo ~ M), mtr_index order
    float* starts;
    int64_t B;              // (packed sequences: the number of sequences)
    int32_t H, dk, dv, n_seg;
    int32_t first;          // 0 or 1 (see above; 0 with seq_table)
    // packed sequences with segments: entry i = {first slot, number of segments} of sequence i;
    // its pairs and starts for head h sit at h * n_seg + first slot + j
    const int2* seq_table;
};

hipError_t launch_scan(const ScanArgs& a, hipStream_t st);

// Segment tables of packed sequences (see ChunkArgs::seg_table, ScanArgs::seq_table): sequence
// i covers tokens [cu[i], cu[i+1]) clamped into [end of sequence i-1, T], cut into segments of
// seg_len tokens (at least one, also when empty); slots past the last segment get sequence -1.
constexpr int SEG_FIRST = 1, SEG_LAST = 2;
struct SegTableArgs {
    const int32_t* cu_seqlens;  // [n_seqs + 1]
    int64_t T, seg_len;
    int32_t n_seqs, n_slots;    // n_slots >= ceil(T / seg_len) + n_seqs
    int4* seg_table;            // [n_slots]
    int2* seq_table;            // [n_seqs]
};

hipError_t launch_seg_table(const SegTableArgs& a, hipStream_t st);

// Position of M[row][k] inside one dk^2 plane of a segment transition: the order in which the
// scan's MFMA reads its A operand, so that each of its loads is one contiguous run of 64 x 16
// bytes.  Mixed radix (16-row tile, 32-deep contraction step, granule g * 16 + m, element),
// where granule (g, m) holds columns 32 t + 8 g .. +7 of row 16 w + m; a (tile, step) pair has
// 16 min(4, dk / 8) granules, so the plane holds exactly dk^2 elements.
// Position of S_loc[row][col] inside one segment's dk x dv block: the order of the accumulator
// tiles (16-column tile, 16-row tile, lane g * 16 + m, element r for row 16 w + 4 g + r, column
// 16 j + m), so that the segment pass stores, and the scan loads, a lane's four rows as one
// 16-byte piece and a wave's tile as one contiguous 1 KiB run.
__host__ __device__ constexpr int sloc_index(int dk, int row, int col) {
    return (((col >> 4) * (dk >> 4) + (row >> 4)) * 64 + ((row >> 2) & 3) * 16 + (col & 15)) * 4 + (row & 3);
}

__host__ __device__ constexpr int mtr_index(int dk, int row, int k) {
    const int ksteps = (dk + 31) / 32, gpt = 16 * (dk / 8 < 4 ? dk / 8 : 4);
    return ((((row >> 4) * ksteps + (k >> 5)) * gpt + ((k >> 3) & 3) * 16 + (row & 15)) << 3) + (k & 7);
}

// ---------------------------------------------------------------- chunk kernel LDS layout
// Byte offsets of the chunk kernel's LDS arrays.  bf16 operands (RV): the A / M tiles take
// their decay factors on the right operand, which is stored in one variant per distance
// between the sub-tiles (RD for the diagonal, RH for adjacent sub-tiles, RF for two and three
// apart).  float32 operands instead scale the left operand in registers by per-channel
// factors (fd, fo), which keeps their LDS footprint small.
struct Lds {
    int kt, qt, kl, ql, rh, rd, rf, kht, an, mm, ad, fd, fo, egc, beta, total;
};

__host__ __device__ constexpr int align16(int x) { return (x + 15) & ~15; }

// E: bytes per operand element
__host__ __device__ constexpr Lds lds_layout(int E, int DK, int C) {
    const bool RV = E == 2;
    const int PADE = 16 / E;
    const int NT = C / 16;
    const int DKP = DK < 32 ? 32 : DK;            // bf16 natural loads read 32 channels at a time
    const int LDK = DKP + PADE;
    const int LKQ = DKP + 4;                      // (the pitches the chunk kernel uses)
    const int LC = C + 4;
    Lds L{};
    int off = 0;
    L.kt = off;   off += align16(C * LKQ * E);
    L.qt = off;   off += align16(C * LKQ * E);
    L.kl = off;   off += align16(C * LDK * E);
    L.ql = off;   off += align16(C * LDK * E);
    L.rh = off;   off += align16(C * LDK * E);
    L.rd = off;   off += RV ? align16(C * LDK * E) : 0;
    L.rf = off;   off += (RV && NT == 4) ? align16(48 * LDK * E) : 0;
    // the Kt..RF region also holds the v staging tile (C rows, up to 128 columns)
    if (off - L.kt < C * (128 + PADE) * E) off = L.kt + align16(C * (128 + PADE) * E);
    L.kht = off;  off += align16(DK * LC * E);
    L.an = off;   off += align16(C * LC * E);
    L.mm = off;   off += align16(C * LC * E);
    L.ad = off;   off += align16(NT * 16 * 16 * 4);
    L.fd = off;   off += RV ? 0 : align16(NT * DKP * 4);
    L.fo = off;   off += RV ? 0 : align16(3 * DKP * 4);
    L.egc = off;  off += align16(2 * DKP * 4);   // two slots: chunk n and chunk n+1
    L.beta = off; off += align16(2 * C * 4);
    L.total = off;
    return L;
}

// Bytes of dynamic LDS the chunk kernel needs for one workgroup.
inline size_t chunk_lds_bytes(bool bf16, int dk, int chunk, int /*dv_block*/) {
    return (size_t)lds_layout(bf16 ? 2 : 4, dk, chunk).total;
}

// ---------------------------------------------------------------- per-lane global offsets
// The chunk kernel addresses a token-major tensor as a 64-bit, wave-uniform base at the
// chunk's first token plus a 32-bit per-lane byte offset (the form scalar-base addressing
// takes, with no 64-bit arithmetic per access).  Token strides are 24-bit products: the ABI
// bounds H * max(dk, dv) below 2^24, and a lane's token lies less than 64 tokens past the
// base, so (tok * stride + col) * esize stays below 63 * (2^24 - 1) * 4 + 512 < 2^32.
__host__ __device__ inline unsigned mul24(unsigned a, unsigned b) {
#if defined(__HIP_DEVICE_COMPILE__)
    return __umul24(a, b);
#else
    return (a & 0xFFFFFFu) * (b & 0xFFFFFFu);     // what v_mul_u32_u24 computes
#endif
}

// element offset of column `col` of token `tok` (tokens `stride` elements apart)
__host__ __device__ inline unsigned tok_elem_off(unsigned tok, unsigned stride, unsigned col) {
    return mul24(tok, stride) + col;
}

// ---------------------------------------------------------------- library-owned workspace
// Address of the current device's copy of the segment workspace that kda_chunk_fwd_noalloc
// uses (KDA_NOALLOC_SCRATCH_BYTES per GPU), looked up once per device.
hipError_t scratch_address(void** out);

}  // namespace kda
