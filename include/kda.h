/*
 * kda.h -- C ABI of the KDA (Kimi Delta Attention) hot-path library for
 * AMD Instinct MI355X (gfx950).  Link with libkda.so.
 *
 * What the library computes.  Per (batch, head) a fixed-size state S with dk
 * rows (key channels) and dv columns (value channels), float32, evolves token
 * by token as
 *
 *     g_t = min(max(log_alpha_t, -5), 0)            per key channel
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * Sources: the state replaces the key/value cache and is updated per token,
 * then multiplied by the query (llm-wiki.hwlabs.dev, "Kimi K3 ... linear
 * attention", section "1. Limits of softmax attention and KDA's direction");
 * one decay gate per feature channel where GatedDeltaNet has one per head
 * (same page, "Difference between GatedDeltaNet and KDA"); log-decay floored
 * so each step keeps at least 0.67 % (orkas.ai "Kimi K3 architecture",
 * section "The floor that removed a GPU code path").  The pages do not print
 * the formula; decay-then-delta order, the post-update read and the clamp at
 * 0 are this library's reading.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor pointers are DEVICE pointers, owned by the caller; the library
 *   never allocates, frees or synchronises.  Work is enqueued on `stream`
 *   (a hipStream_t; NULL = the default stream).  KDA_OK means "enqueued".
 * - Layouts are dense row-major (C order), base pointers 16-byte aligned.
 * - Argument errors are detected before any HIP call: the call returns the
 *   code, writes nothing and records a message for kda_last_error().  Input
 *   values are not checked: NaN / Inf propagate.  (Device-side arrays, such
 *   as cu_seqlens and n_accept, are read on the device: see each call.)
 * - A failed kernel launch returns KDA_ERR_HIP (text via kda_last_error()).
 * - Supported sizes: dk, dv in {16, 32, 64, 128}; chunk in {16, 32, 64};
 *   any T >= 0 (a partial last chunk is masked); B, N, H >= 1 with
 *   H * max(dk, dv) < 2^24 (token strides are formed as 24-bit products).  For
 *   float32 q/k/v the chunk must satisfy chunk * dk <= 4096 (LDS capacity).
 * - Thread safety: calls are reentrant; concurrent calls on one stream run in
 *   stream order, calls on different streams must not share output buffers.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 2

/* Storage type of q, k, v and o.  log_alpha, beta and every state are float32.
 * (KDA_DTYPE_FORCE_INT32 is not a dtype: it makes every non-negative int32 a valid value of
 * the type, so an unknown code passed from C is rejected with KDA_ERR_DTYPE rather than being
 * an out-of-range enum value in the library's C++.) */
typedef enum { KDA_DTYPE_F32 = 0, KDA_DTYPE_BF16 = 1, KDA_DTYPE_FORCE_INT32 = 0x7fffffff } kda_dtype_t;

/* Input options of every call, bit flags (kda_plan_t.flags for kda_chunk_fwd, the `flags`
 * argument of the decode calls); 0 = none.
 * KDA_GATE_LOGITS: log_alpha holds raw gate logits x; the log-decay is the floored
 *   activation -5 sigmoid(x) = -5 / (1 + e^-x), in (-5, 0), computed inside the kernels
 *   (the floor constant is what made the gate's activation need a lower bound: orkas.ai
 *   "Kimi K3 architecture", section "The floor that removed a GPU code path"; the
 *   sigmoid form is this library's reading).  Same bytes read, no separate pass.
 * KDA_QK_L2NORM: q and k are normalised per token and head inside the kernels,
 *   x / sqrt(sum_c x_c^2 + 1e-6) over the dk channels, before every other step.  The
 *   pages leave normalisation to the model; the epsilon form is this library's choice. */
typedef enum { KDA_GATE_LOGITS = 1, KDA_QK_L2NORM = 2 } kda_input_flag_t;

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL = 1,          /* a required pointer is NULL                       */
    KDA_ERR_SHAPE = 2,         /* a size is negative / zero where it must not be   */
    KDA_ERR_DTYPE = 3,         /* unknown dtype enum                               */
    KDA_ERR_ALIGN = 4,         /* a pointer is not 16-byte aligned                  */
    KDA_ERR_UNSUPPORTED = 5,   /* dk / dv / chunk / plan outside the supported set  */
    KDA_ERR_WORKSPACE = 6,     /* workspace missing or smaller than required        */
    KDA_ERR_HIP = 7,           /* the HIP runtime reported an error                 */
    KDA_ERR_ALIAS = 8,         /* an output overlaps an input it must not alias     */
    KDA_STATUS_FORCE_INT32 = 0x7fffffff   /* not a status: widens the type (see kda_dtype_t) */
} kda_status_t;

/*
 * Execution plan of kda_chunk_fwd.
 *
 * n_segments: split each sequence into this many token segments (each a whole
 *   number of chunks).  1 = one sequential pass.  > 1 = the segment
 *   decomposition of orkas.ai "Kimi K3 architecture", section "The cost comes
 *   back in the serving stack": pass 1 builds every segment's (cumulative
 *   transition, zero-start state) pair, a prefix scan gives each segment's
 *   true start state, pass 2 reruns the segments in parallel from those.
 * seg0_len: 0 = segments of equal length.  > 0 (unpacked batches, n_segments
 *   >= 2) = the lead form: segment 0 holds seg0_len tokens (a multiple of
 *   chunk, below T) and the other T - seg0_len tokens are cut into
 *   n_segments - 1 equal segments of whole chunks.  Segment 0 needs no scan (it
 *   starts from S0), so it runs in pass-2 form in the same launch as pass 1 over
 *   segments 1 .. n_segments - 2, on the compute units that pass 1 leaves
 *   free; its final state is the exact start of segment 1, and the scan and
 *   pass 2 cover segments 1 .. n_segments - 1.  Results equal those of equal
 *   segments up to rounding.
 * dv_block: value columns per workgroup of the one-pass / pass-2 launch, a
 *   multiple of 16 dividing dv.  The recurrence is independent per state
 *   column, so column blocks run in parallel; the shared per-chunk work
 *   (gates, WY transform) is repeated per block.  Pass 1 of a segmented plan
 *   always holds all dv + dk columns of its widened state in one workgroup.
 * state_ckpt / ckpt_stride: optional state checkpoints for prefix reuse
 *   (orkas.ai "Kimi K3 architecture", section "The cost comes back in the
 *   serving stack": the recurrent state is checkpointed sparsely, at some of
 *   the 512-token hash boundaries, so a cache hit can restore it).  When
 *   state_ckpt is not NULL, ckpt_stride is a positive multiple of chunk and
 *   state_ckpt [B, T / ckpt_stride (rounded down), H, dk, dv] float32 receives
 *   the state after tokens ckpt_stride, 2 ckpt_stride, ... of each sequence
 *   (the start state S0 counts as the state before token 0).  It must be
 *   16-byte aligned and overlap no other argument.  NULL = no checkpoints.
 * cu_seqlens / n_seqs: optional packed variable-length batch.  When
 *   cu_seqlens is not NULL the call takes B == 1 and n_seqs sequences packed
 *   along T: sequence i owns tokens [cu_seqlens[i], cu_seqlens[i+1]) (device
 *   int32 array of n_seqs + 1 nondecreasing offsets from 0 to T; chunks start
 *   at each sequence's first token), and S0 / S_T are [n_seqs, H, dk, dv].  No
 *   state checkpoints.  The offsets are read on the device: values outside
 *   [0, T] are clamped, other invalid arrays give unspecified (but in-bounds)
 *   results.  With packed sequences n_segments > 1 cuts the packed row into
 *   that many segments: every sequence is split into segments of
 *   ceil(T / n_segments) tokens (rounded up to whole chunks, at least two
 *   chunks), so only sequences longer than that are split, each with its own
 *   prefix scan; 0 = one pass when the (sequence, head, column block) units
 *   cover MI355X's 256 compute units or T is shorter than 8 chunks, else
 *   floor(256 / (H x column blocks)) segments, one round of workgroups
 *   (needs T < 2^31; the segment tables are built on the device from
 *   cu_seqlens inside the workspace).
 * flags: kda_input_flag_t bits (0 = log-decays, q and k used as given).
 * A zeroed plan (all fields 0 / NULL) means "library default" for each field.
 */
typedef struct {
    int32_t n_segments;
    int32_t dv_block;
    /* Optional launch timing, for profilers and benchmarks (NULL = off).  An
     * array of n_launch_events hipEvent_t handles, created by the caller.
     * Kernel launch i of the call (i = 0, 1, ... in launch order: one launch
     * with one segment; pass 1, scan, pass 2 with several; lead (segment 0
     * beside pass 1), scan, pass 2 in the lead form, without the scan when
     * n_segments is 2; the segment-table build first for packed sequences with
     * segments) records
     * launch_events[2i] just before it and launch_events[2i+1] just after it
     * on `stream`; launches beyond the array's capacity record nothing. */
    void* const* launch_events;
    int32_t n_launch_events;
    float* state_ckpt;
    int64_t ckpt_stride;
    const int32_t* cu_seqlens;
    int32_t n_seqs;
    uint32_t flags;
    int64_t seg0_len;
} kda_plan_t;

/* Fills *plan with the library's default for this problem: one pass when the
 * (batch, head) units alone leave fewer than half of MI355X's 256 compute units
 * idle (units > 128) or the sequence is shorter than 8 chunks, otherwise
 * floor(256 / units) segments (at least two chunks per segment), so that each
 * launch fits one round of workgroups (a chunk
 * workgroup of dk = 128 fills a CU's LDS, and a launch of more workgroups than
 * CUs runs the excess in a second round).  The default takes
 * the lead form (seg0_len) when, counting a pass-1 chunk as 0.8 of a pass-2
 * chunk's time (as measured on MI355X), it is at least 2 % shorter than the
 * equal segments: one more segment, segment 0 sized so that the launch running
 * it beside pass 1 ends together.  The default is
 * the same on every device (it does not query the device), so results round
 * the same everywhere; on a partitioned device pass n_segments yourself.
 * Returns KDA_OK or an argument error.  Makes no HIP call.
 * With KDA_TRACE=1 in the environment, every kda_chunk_fwd call prints its
 * resolved plan (segments, segment length, column block, workspace, launches)
 * to stderr. */
kda_status_t kda_chunk_fwd_default_plan(int64_t B, int64_t T, int32_t H, int32_t dk,
                                        int32_t dv, int32_t chunk, kda_dtype_t dt,
                                        kda_plan_t* plan);

/* Device workspace, in bytes, that kda_chunk_fwd needs for this problem and
 * plan (plan NULL = default plan).  0 when the plan has one segment. */
kda_status_t kda_chunk_fwd_workspace_bytes(int64_t B, int64_t T, int32_t H, int32_t dk,
                                           int32_t dv, int32_t chunk, kda_dtype_t dt,
                                           const kda_plan_t* plan, size_t* bytes);

/*
 * Chunked prefill: the recurrence above over T tokens per sequence, evaluated
 * chunk by chunk.  Within a chunk the decays enter as ratios of cumulative
 * decays; the floor keeps a 16-token tile's cumulative log-decay in [-80, 0],
 * so every intra-chunk tile, the diagonal ones included, is an ordinary dense
 * matrix product (orkas.ai "Kimi K3 architecture", section "The floor that
 * removed a GPU code path").  With n_segments > 1 the sequence is split into
 * (cumulative transition, zero-start state) pairs composed by a prefix scan
 * (same page, section "The cost comes back in the serving stack").  The
 * result does not depend on chunk or plan beyond rounding.
 *
 *   q, k       [B, T, H, dk]  dt
 *   v          [B, T, H, dv]  dt
 *   log_alpha  [B, T, H, dk]  float32 log-decays (values outside [-5, 0] are clamped),
 *              or raw gate logits when plan->flags has KDA_GATE_LOGITS
 *   beta       [B, T, H]      float32
 *   S0         [B, H, dk, dv] float32 start state, or NULL for zeros
 *   o          [B, T, H, dv]  dt, written
 *   S_T        [B, H, dk, dv] float32 final state, written; may equal S0
 *              (advance in place) but must not partially overlap it
 *   chunk      tokens per chunk (16, 32 or 64); changes rounding, not the result
 *   plan       NULL = default, else an explicit plan (see kda_plan_t)
 *   workspace  device scratch of at least kda_chunk_fwd_workspace_bytes();
 *              may be NULL when that size is 0.  Its contents are not needed
 *              before or after the call.
 *
 * o must not overlap any input.  With T == 0 the call copies S0 (or zeros)
 * into S_T and writes no o.
 */
kda_status_t kda_chunk_fwd(const void* q, const void* k, const void* v,
                           const float* log_alpha, const float* beta, const float* S0,
                           void* o, float* S_T,
                           int64_t B, int64_t T, int32_t H, int32_t dk, int32_t dv,
                           int32_t chunk, kda_dtype_t dt, const kda_plan_t* plan,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc.  Same
 * arguments, meaning and errors as kda_chunk_fwd except that there is no
 * workspace argument: a segmented plan uses a segment workspace the library
 * owns, one array of KDA_NOALLOC_SCRATCH_BYTES per GPU, kept until the
 * process ends.  The call itself allocates nothing.
 *
 * - A plan whose segment workspace (kda_chunk_fwd_workspace_bytes) exceeds
 *   KDA_NOALLOC_SCRATCH_BYTES is rejected with KDA_ERR_WORKSPACE before any
 *   HIP call.  The default plans of B=1, T=4096, H=16 (16 segments) and of
 *   B=1, T=1,048,576, H=32 (9 segments in the lead form), dk = dv = 128, need
 *   48 and 54 MiB.
 * - On the first call on a device that needs the array, the library looks up
 *   its address on that device (hipGetSymbolAddress); a failure there returns
 *   KDA_ERR_HIP.
 * - Every call on one GPU shares that GPU's array: calls that may overlap in
 *   time on one GPU (different streams, different host threads) race and give
 *   undefined results.  Calls ordered on one stream are safe.  No part of the
 *   array needs to start at zero: a call reads only what it wrote earlier.
 */
#define KDA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

kda_status_t kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                   const float* log_alpha, const float* beta, const float* S0,
                                   void* o, float* S_T,
                                   int64_t B, int64_t T, int32_t H, int32_t dk, int32_t dv,
                                   int32_t chunk, kda_dtype_t dt, const kda_plan_t* plan,
                                   void* stream);

/*
 * One recurrent decode step for N independent sequences, state updated in
 * place (orkas.ai "Kimi K3 architecture", section "The cost comes back in the
 * serving stack": the state is updated in place).  Equivalent to
 * kda_chunk_fwd with T = 1 and S_T == S0.
 *
 *   state      [N, H, dk, dv] float32, read and overwritten
 *   q, k       [N, H, dk]     dt
 *   v          [N, H, dv]     dt
 *   log_alpha  [N, H, dk]     float32, read as `flags` says
 *   beta       [N, H]         float32
 *   o          [N, H, dv]     dt, written; must not overlap state or inputs
 * Sizes: dk, dv in {16, 32, 64, 128}; N * H < 2^31.
 */
kda_status_t kda_decode_step(float* state, const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta, void* o,
                             int64_t N, int32_t H, int32_t dk, int32_t dv, kda_dtype_t dt,
                             uint32_t flags, void* stream);

/*
 * Speculative decoding, verify half.  Because the state is updated in place, a
 * rejected draft could not be rolled back (orkas.ai "Kimi K3 architecture",
 * section "The cost comes back in the serving stack"): this call evaluates
 * n_draft draft tokens per sequence from `state` WITHOUT writing it.  o for
 * draft j is the output after drafts 0..j, i.e. what n_draft successive
 * kda_decode_step calls would return.
 *
 *   state      [N, H, dk, dv]       float32, read only
 *   q, k       [N, n_draft, H, dk]  dt
 *   v          [N, n_draft, H, dv]  dt
 *   log_alpha  [N, n_draft, H, dk]  float32, read as `flags` says
 *   beta       [N, n_draft, H]      float32
 *   o          [N, n_draft, H, dv]  dt, written; must not overlap any input
 * Sizes: as kda_decode_step, 1 <= n_draft and N * n_draft * H < 2^31.
 */
kda_status_t kda_decode_verify(const float* state, const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta, void* o,
                               int64_t N, int32_t n_draft, int32_t H, int32_t dk, int32_t dv,
                               kda_dtype_t dt, uint32_t flags, void* stream);

/*
 * Speculative decoding, commit half (same section): the caller keeps the drafts'
 * per-token inputs (q, k, v, log_alpha, beta: a few hundred bytes per token and
 * head, against the state's dk * dv * 4) and, once n_accept[n] of sequence n's
 * drafts are accepted, this call replays them on the GPU: state[n] advances by
 * drafts 0 .. n_accept[n]-1, exactly as that many kda_decode_step calls would.
 *
 *   state      [N, H, dk, dv] float32, read and overwritten
 *   q, k, v, log_alpha, beta   as kda_decode_verify (the same buffers)
 *   n_accept   [N] int32 DEVICE array, 4-byte aligned; read on the device, values
 *              clamped to [0, n_draft] (0 leaves that sequence's state unchanged)
 * The state must not overlap any input or n_accept.
 */
kda_status_t kda_decode_commit(float* state, const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta, const int32_t* n_accept,
                               int64_t N, int32_t n_draft, int32_t H, int32_t dk, int32_t dv,
                               kda_dtype_t dt, uint32_t flags, void* stream);

/* Static description of a status code. */
const char* kda_status_str(kda_status_t status);

/* Text of the last error recorded on the calling thread ("" if none). */
const char* kda_last_error(void);

/* KDA_ABI_VERSION of the loaded library. */
int32_t kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
