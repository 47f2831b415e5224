// C ABI of libkda.so: argument validation, plan selection and launch order.
// Every argument error is detected before the first HIP call.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "kda.h"
#include "kda_internal.h"

namespace {

thread_local char g_err[512] = "";

kda_status_t fail(kda_status_t s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

kda_status_t hip_fail(hipError_t e, const char* what) {
    return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool dim_ok(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool chunk_ok(int32_t c) { return c == 16 || c == 32 || c == 64; }
bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
constexpr uint32_t kAllFlags = KDA_GATE_LOGITS | KDA_QK_L2NORM;

// Compute units the default plan is sized for: MI355X (gfx950) has 256.  A constant, not a
// device query: the default plan, and with it the rounding of the results, is the same on
// every device, and no HIP call is needed before the arguments are validated.  Callers on a
// partitioned device pass n_segments themselves.
constexpr int64_t kPlanCUs = 256;

// KDA_TRACE=1 in the environment: every kda_chunk_fwd call prints its resolved plan to stderr.
bool trace_on() {
    static const bool on = [] {
        const char* e = std::getenv("KDA_TRACE");
        return e && *e && std::strcmp(e, "0") != 0;
    }();
    return on;
}

kda_status_t check_problem(int64_t B, int64_t T, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                           kda_dtype_t dt) {
    if (B < 1 || H < 1 || T < 0) return fail(KDA_ERR_SHAPE, "need B >= 1, H >= 1, T >= 0 (got B=%lld H=%d T=%lld)",
                                             (long long)B, H, (long long)T);
    if (dt != KDA_DTYPE_F32 && dt != KDA_DTYPE_BF16) return fail(KDA_ERR_DTYPE, "unknown dtype %d", (int)dt);
    if (!dim_ok(dk) || !dim_ok(dv)) return fail(KDA_ERR_UNSUPPORTED, "dk, dv must be 16, 32, 64 or 128 (got %d, %d)", dk, dv);
    if (!chunk_ok(chunk)) return fail(KDA_ERR_UNSUPPORTED, "chunk must be 16, 32 or 64 (got %d)", chunk);
    if (dt == KDA_DTYPE_F32 && chunk * dk > 4096)
        return fail(KDA_ERR_UNSUPPORTED, "float32 inputs need chunk * dk <= 4096 (got %d)", chunk * dk);
    if (B * T * (int64_t)H > (int64_t)1 << 40) return fail(KDA_ERR_SHAPE, "problem too large");
    if ((int64_t)H * (dk > dv ? dk : dv) >= (int64_t)1 << 24)   // token strides are 24-bit products
        return fail(KDA_ERR_UNSUPPORTED, "H * max(dk, dv) must be below 2^24 (got H=%d)", H);
    return KDA_OK;
}

struct Resolved {
    int32_t n_seg;          // segments per sequence; packed sequences: slots of the segment table
    int64_t seg_len;        // tokens per segment, a multiple of the chunk
    int32_t dv_block;
    bool packed_seg;        // packed sequences cut into segments (segment tables in the workspace)
    int32_t n_seqs;         // packed sequences (0 without cu_seqlens)
    int64_t seg0_len;       // lead form: tokens of segment 0 (0 = equal segments)
};

// Default lead form: a pass-1 chunk (the widened state [S | M], no q, no o) takes about this
// fraction r of a pass-2 chunk's time on MI355X (bf16, 128 x 128: 6.0 vs 7.5 us in the 1M-token
// plan; a sweep of segment 0's length there had its optimum at this ratio).  In pass-2-chunk
// units, S equal segments of L chunks cost L (1 + r) (pass 1, then pass 2); the lead form with S
// segments of l chunks after a segment 0 of c0 = chunks - S l costs max(c0, r l) + l (segment
// 0 beside pass 1, then pass 2).  The default takes the lead form when that is at least
// kLeadGain cheaper, with l the better of the two whole numbers around chunks / (S + r).
constexpr double kLeadRatio = 0.8;
// Sequences shorter than this many chunks run in one pass: the two extra launches of a
// segmented plan (pass 1 and the scan) cost more than they save below it (MI355X, dk = dv = 128,
// chunk 64, one sequence x 8 or 32 heads: 4 chunks 33-34 us in one pass against 42-46 us in 2
// segments; 8 chunks 59-60 us against 46-51 us in 4 segments).
constexpr int64_t kMinChunksToSplit = 8;
constexpr double kLeadGain = 0.98;

constexpr int64_t kMaxSlots = 1 << 22;   // segment-table entries of one packed call

kda_status_t resolve_plan(int64_t B, int64_t T, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                          kda_dtype_t dt, const kda_plan_t* plan, Resolved* out) {
    kda_plan_t p = plan ? *plan : kda_plan_t{};
    int32_t dvb = p.dv_block;
    if (dvb == 0) dvb = dv;                                   // one column block per (b, h)
    if (dvb < 16 || dvb > 128 || dvb % 16 != 0 || dv % dvb != 0)
        return fail(KDA_ERR_UNSUPPORTED, "dv_block %d must be a multiple of 16 that divides dv=%d, at most 128", dvb, dv);
    if (kda::chunk_lds_bytes(dt == KDA_DTYPE_BF16, dk, chunk, dvb) > 163840)
        return fail(KDA_ERR_UNSUPPORTED, "dk=%d chunk=%d dv_block=%d exceeds the 160 KiB LDS of a workgroup", dk, chunk, dvb);
    const int64_t nchunks = (T + chunk - 1) / chunk;
    int64_t nseg = p.n_segments;
    if (nseg < 0) return fail(KDA_ERR_UNSUPPORTED, "n_segments must be >= 0");
    out->packed_seg = false;
    out->n_seqs = 0;
    out->dv_block = dvb;
    out->seg0_len = 0;
    if (p.seg0_len < 0) return fail(KDA_ERR_UNSUPPORTED, "seg0_len must be >= 0");
    if (p.seg0_len > 0 && p.cu_seqlens) return fail(KDA_ERR_UNSUPPORTED, "seg0_len applies to unpacked batches only");
    if (p.cu_seqlens) {
        // Packed sequences: n_segments is the number of segments the packed row is cut into;
        // every sequence is split into segments of that length (whole chunks, at least two), so
        // only the sequences longer than it are split.  Default: one pass when the (sequence,
        // head, column block) units cover the compute units or the packed row is shorter than
        // kMinChunksToSplit chunks, else as many segments as one round of workgroups holds (as
        // below).
        const int64_t ns = p.n_seqs;
        if (ns < 1) return fail(KDA_ERR_SHAPE, "n_seqs must be >= 1 (got %lld)", (long long)ns);
        out->n_seqs = (int32_t)ns;
        const int64_t per_slot = (int64_t)H * (dv / dvb);
        if (nseg == 0) nseg = ns * per_slot < kPlanCUs && nchunks >= kMinChunksToSplit ? kPlanCUs / per_slot : 1;
        int64_t seg_chunks = nchunks == 0 ? 1 : (nchunks + nseg - 1) / nseg;
        if (seg_chunks < 2) seg_chunks = 2;
        if (nseg > 1 && seg_chunks < nchunks) {
            if (T >= ((int64_t)1 << 31)) return fail(KDA_ERR_UNSUPPORTED, "packed sequences with segments need T < 2^31");
            const int64_t seg_len = seg_chunks * chunk;
            const int64_t slots = (T + seg_len - 1) / seg_len + ns;
            if (slots > kMaxSlots) return fail(KDA_ERR_UNSUPPORTED, "too many segments for packed sequences");
            out->packed_seg = true;
            out->n_seg = (int32_t)slots;
            out->seg_len = seg_len;
            return KDA_OK;
        }
        out->n_seg = 1;
        out->seg_len = nchunks * chunk;
        return KDA_OK;
    }
    if (p.seg0_len > 0) {
        // the lead form as asked: segment 0 of seg0_len tokens, the rest in nseg - 1 segments
        if (p.seg0_len % chunk != 0 || p.seg0_len >= T)
            return fail(KDA_ERR_UNSUPPORTED, "seg0_len (%lld) must be a multiple of chunk (%d) below T (%lld)",
                        (long long)p.seg0_len, chunk, (long long)T);
        if (nseg < 2) return fail(KDA_ERR_UNSUPPORTED, "seg0_len needs n_segments >= 2 (got %lld)", (long long)nseg);
        if (nseg > 65535) return fail(KDA_ERR_UNSUPPORTED, "too many segments");
        const int64_t rest = nchunks - p.seg0_len / chunk;           // >= 1
        const int64_t lc = (rest + nseg - 2) / (nseg - 1);
        out->seg0_len = p.seg0_len;
        out->seg_len = lc * chunk;
        out->n_seg = (int32_t)(1 + (rest + lc - 1) / lc);
        return KDA_OK;
    }
    const bool dflt = nseg == 0;
    if (nseg == 0) {
        // as many segments as fit the compute units in one round of workgroups (one workgroup
        // of the 128 x 128 chunk kernel fills a CU's LDS, so a launch of more than kPlanCUs
        // workgroups runs the excess in a second round); segments only when (b, h, column
        // block) units alone leave CUs idle, only for sequences of kMinChunksToSplit chunks or
        // more, and only if each segment keeps at least 2 chunks
        const int64_t units = B * H * (dv / dvb);
        const int64_t cus = kPlanCUs;
        nseg = 1;
        if (units < cus && nchunks >= kMinChunksToSplit) {
            nseg = cus / units;
            if (nseg > nchunks / 2) nseg = nchunks / 2;
            if (nseg < 1) nseg = 1;
        }
    }
    if (nseg > 65535) return fail(KDA_ERR_UNSUPPORTED, "too many segments");
    int64_t seg_chunks = nchunks == 0 ? 1 : (nchunks + nseg - 1) / nseg;
    if (seg_chunks < 1) seg_chunks = 1;
    out->seg_len = seg_chunks * chunk;
    out->n_seg = nchunks == 0 ? 1 : (int32_t)((nchunks + seg_chunks - 1) / seg_chunks);
    out->dv_block = dvb;
    if (dflt && out->n_seg >= 2) {
        // lead form: one segment more, segment 0 sized so that the launch running it beside
        // pass 1 ends together, and pass 2 covering one segment fewer (cost model above)
        const int64_t S = nseg;                                     // pass-2 workgroups per unit
        const double r = kLeadRatio;
        double best = (double)seg_chunks * (1.0 + r) * kLeadGain;
        int64_t best_l = 0;
        const int64_t lf = (int64_t)((double)nchunks / ((double)S + r));
        for (int64_t l = lf; l <= lf + 1; ++l) {
            const int64_t c0 = nchunks - S * l;
            if (l < 2 || c0 < 1) continue;
            const double cost = ((double)c0 > r * (double)l ? (double)c0 : r * (double)l) + (double)l;
            if (cost < best) {
                best = cost;
                best_l = l;
            }
        }
        if (best_l > 0) {
            out->seg0_len = (nchunks - S * best_l) * chunk;
            out->seg_len = best_l * chunk;
            out->n_seg = (int32_t)(S + 1);
        }
    }
    return KDA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Segment workspace: S_loc, M (two bf16 planes, the bytes of one float plane) and the start
// states of every (sequence or slot, head, segment), then the segment tables of packed sequences.
size_t workspace_for(int64_t B, int32_t H, int32_t dk, int32_t dv, const Resolved& r) {
    if (r.n_seg <= 1 && !r.packed_seg) return 0;
    size_t n = (size_t)B * H * r.n_seg * ((size_t)2 * dk * dv + (size_t)dk * dk) * sizeof(float);
    if (r.packed_seg) n = align256(n) + align256((size_t)r.n_seg * 16) + (size_t)r.n_seqs * 8;
    return n;
}

// Records the caller's timing events around each kernel launch of one call.
struct LaunchEvents {
    void* const* ev;
    int32_t n;
    int32_t i;
    hipStream_t st;
    void before() {
        if (ev && 2 * i + 1 < n) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(ev[2 * i]), st);
    }
    void after() {
        if (ev && 2 * i + 1 < n) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(ev[2 * i + 1]), st);
        ++i;
    }
};

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

const char* kda_status_str(kda_status_t s) {
    switch (s) {
        case KDA_OK: return "ok";
        case KDA_ERR_NULL: return "null pointer";
        case KDA_ERR_SHAPE: return "invalid shape";
        case KDA_ERR_DTYPE: return "invalid dtype";
        case KDA_ERR_ALIGN: return "pointer not 16-byte aligned";
        case KDA_ERR_UNSUPPORTED: return "unsupported size or plan";
        case KDA_ERR_WORKSPACE: return "workspace too small";
        case KDA_ERR_HIP: return "HIP runtime error";
        case KDA_ERR_ALIAS: return "output overlaps an input";
        default: break;
    }
    return "unknown status";
}

const char* kda_last_error(void) { return g_err; }

int32_t kda_abi_version(void) { return KDA_ABI_VERSION; }

kda_status_t kda_chunk_fwd_default_plan(int64_t B, int64_t T, int32_t H, int32_t dk, int32_t dv,
                                        int32_t chunk, kda_dtype_t dt, kda_plan_t* plan) {
    if (!plan) return fail(KDA_ERR_NULL, "plan is NULL");
    kda_status_t s = check_problem(B, T, H, dk, dv, chunk, dt);
    if (s != KDA_OK) return s;
    Resolved r;
    s = resolve_plan(B, T, H, dk, dv, chunk, dt, nullptr, &r);
    if (s != KDA_OK) return s;
    *plan = kda_plan_t{};
    plan->n_segments = r.n_seg;
    plan->dv_block = r.dv_block;
    plan->seg0_len = r.seg0_len;
    return KDA_OK;
}

kda_status_t kda_chunk_fwd_workspace_bytes(int64_t B, int64_t T, int32_t H, int32_t dk, int32_t dv,
                                           int32_t chunk, kda_dtype_t dt, const kda_plan_t* plan,
                                           size_t* bytes) {
    if (!bytes) return fail(KDA_ERR_NULL, "bytes is NULL");
    kda_status_t s = check_problem(B, T, H, dk, dv, chunk, dt);
    if (s != KDA_OK) return s;
    Resolved r;
    s = resolve_plan(B, T, H, dk, dv, chunk, dt, plan, &r);
    if (s != KDA_OK) return s;
    *bytes = workspace_for(B, H, dk, dv, r);
    return KDA_OK;
}

}  // extern "C"

namespace {

// Address of the current device's copy of the library's segment workspace (kda_scratch.hip),
// or null with a message.
void* scratch_address() {
    void* p = nullptr;
    const hipError_t e = kda::scratch_address(&p);
    if (e != hipSuccess) {
        hip_fail(e, "segment workspace address");
        return nullptr;
    }
    return p;
}

// kda_chunk_fwd and kda_chunk_fwd_noalloc: with `library_scratch` the segment workspace is the
// library's own array (workspace / workspace_bytes are ignored).
kda_status_t chunk_fwd_impl(const void* q, const void* k, const void* v, const float* log_alpha,
                            const float* beta, const float* S0, void* o, float* S_T, int64_t B,
                            int64_t T, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                            kda_dtype_t dt, const kda_plan_t* plan, void* workspace,
                            size_t workspace_bytes, void* stream, bool library_scratch) {
    kda_status_t s = check_problem(B, T, H, dk, dv, chunk, dt);
    if (s != KDA_OK) return s;
    if (!S_T) return fail(KDA_ERR_NULL, "S_T is NULL");
    if (T > 0 && (!q || !k || !v || !log_alpha || !beta || !o))
        return fail(KDA_ERR_NULL, "q, k, v, log_alpha, beta and o are required when T > 0");
    const int32_t* cu = plan ? plan->cu_seqlens : nullptr;
    const int64_t n_seq = cu ? plan->n_seqs : B;            // state rows: sequences
    if (cu) {
        if (B != 1) return fail(KDA_ERR_SHAPE, "packed sequences (cu_seqlens) need B == 1 (got %lld)", (long long)B);
        if (plan->n_seqs < 1) return fail(KDA_ERR_SHAPE, "n_seqs must be >= 1 (got %d)", plan->n_seqs);
        if (reinterpret_cast<uintptr_t>(cu) % 4 != 0) return fail(KDA_ERR_ALIGN, "cu_seqlens is not 4-byte aligned");
        if (plan->state_ckpt) return fail(KDA_ERR_UNSUPPORTED, "state checkpoints are not available with cu_seqlens");
    }
    const uint32_t flags = plan ? plan->flags : 0u;
    if (flags & ~kAllFlags) return fail(KDA_ERR_UNSUPPORTED, "unknown input flags 0x%x", flags);
    float* ckpt = plan ? plan->state_ckpt : nullptr;
    const int64_t ckpt_stride = ckpt ? plan->ckpt_stride : 0;
    if (ckpt && (ckpt_stride <= 0 || ckpt_stride % chunk != 0))
        return fail(KDA_ERR_UNSUPPORTED, "ckpt_stride (%lld) must be a positive multiple of chunk (%d)",
                    (long long)ckpt_stride, chunk);
    const void* ptrs[] = {q, k, v, log_alpha, beta, S0, o, S_T, workspace, ckpt};
    for (const void* p : ptrs)
        if (p && !aligned(p)) return fail(KDA_ERR_ALIGN, "pointer %p is not 16-byte aligned", p);
    Resolved r;
    s = resolve_plan(B, T, H, dk, dv, chunk, dt, plan, &r);
    if (s != KDA_OK) return s;
    const size_t need = workspace_for(B, H, dk, dv, r);
    if (library_scratch) {
        if (need > KDA_NOALLOC_SCRATCH_BYTES)
            return fail(KDA_ERR_WORKSPACE, "this plan needs %zu bytes of segment workspace; the library holds %zu",
                        need, (size_t)KDA_NOALLOC_SCRATCH_BYTES);
        workspace = nullptr;
        workspace_bytes = 0;
    } else if (need > 0 && (!workspace || workspace_bytes < need)) {
        return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : (size_t)0);
    }

    const size_t es = dt == KDA_DTYPE_BF16 ? 2 : 4;
    const size_t n_qk = (size_t)(B * T * H) * dk, n_v = (size_t)(B * T * H) * dv;
    const size_t n_s = (size_t)(n_seq * H) * dk * dv * 4;
    const size_t n_o = n_v * es;
    struct Span { const void* p; size_t n; const char* name; } ins[] = {
        {q, n_qk * es, "q"}, {k, n_qk * es, "k"}, {v, n_v * es, "v"}, {log_alpha, n_qk * 4, "log_alpha"},
        {beta, (size_t)(B * T * H) * 4, "beta"}, {S0, S0 ? n_s : 0, "S0"}, {S_T, n_s, "S_T"},
        {workspace, need, "workspace"}};
    for (const Span& in : ins)
        if (T > 0 && overlaps(o, n_o, in.p, in.n)) return fail(KDA_ERR_ALIAS, "o overlaps %s", in.name);
    for (int i = 0; i < 5; ++i)
        if (overlaps(S_T, n_s, ins[i].p, ins[i].n)) return fail(KDA_ERR_ALIAS, "S_T overlaps %s", ins[i].name);
    if (S0 && S0 != S_T && overlaps(S0, n_s, S_T, n_s)) return fail(KDA_ERR_ALIAS, "S_T partially overlaps S0");
    if (need > 0) {
        for (int i = 0; i < 7; ++i)
            if (overlaps(workspace, need, ins[i].p, ins[i].n)) return fail(KDA_ERR_ALIAS, "workspace overlaps %s", ins[i].name);
    }
    if (ckpt) {
        const size_t n_ck = (size_t)(T / ckpt_stride) * n_s;
        for (const Span& in : ins)
            if (overlaps(ckpt, n_ck, in.p, in.n)) return fail(KDA_ERR_ALIAS, "state_ckpt overlaps %s", in.name);
        if (T > 0 && overlaps(ckpt, n_ck, o, n_o)) return fail(KDA_ERR_ALIAS, "state_ckpt overlaps o");
    }

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (plan && plan->launch_events && plan->n_launch_events < 0)
        return fail(KDA_ERR_UNSUPPORTED, "n_launch_events must be >= 0");
    if (library_scratch && need > 0) {
        workspace = scratch_address();
        if (!workspace) return KDA_ERR_HIP;
    }
    LaunchEvents tm{plan ? plan->launch_events : nullptr, plan ? plan->n_launch_events : 0, 0, st};
    kda::ChunkArgs a{};
    a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta;
    a.o = o; a.s_final = S_T;
    a.B = B; a.T = T; a.H = H; a.dk = dk; a.dv = dv; a.chunk = chunk;
    a.n_seg = r.n_seg; a.seg_len = r.seg_len; a.seg0_len = r.seg0_len; a.dv_block = r.dv_block;
    a.ckpt = ckpt; a.ckpt_stride = ckpt_stride;
    a.cu_seqlens = cu;
    a.flags = flags;
    if (cu) a.B = n_seq;                      // units and state rows are sequences
    a.bf16 = dt == KDA_DTYPE_BF16;
    if (trace_on()) {
        std::fprintf(stderr,
                     "kda_chunk_fwd%s: B=%lld T=%lld H=%d dk=%d dv=%d chunk=%d dtype=%s sequences=%lld "
                     "%s=%d seg_len=%lld seg0_len=%lld dv_block=%d workspace=%zu flags=0x%x checkpoints=%s "
                     "launches=%s\n",
                     library_scratch ? "_noalloc" : "", (long long)B, (long long)T, H, dk, dv, chunk,
                     dt == KDA_DTYPE_BF16 ? "bf16" : "f32", (long long)n_seq,
                     r.packed_seg ? "segment_slots" : "n_segments", r.n_seg, (long long)r.seg_len,
                     (long long)r.seg0_len, r.dv_block, need, flags, ckpt ? "yes" : "no",
                     r.packed_seg ? "segment-table,segment-pass-1,scan,segment-pass-2"
                     : r.seg0_len > 0 ? (r.n_seg > 2 ? "lead(segment-0+segment-pass-1),scan,segment-pass-2"
                                                     : "lead(segment-0),segment-pass-2")
                     : (r.n_seg == 1 ? "chunk" : "segment-pass-1,scan,segment-pass-2"));
    }
    hipError_t e;
    if (r.n_seg == 1 && !r.packed_seg) {
        a.mode = 0;
        a.s0 = S0;
        a.seg_lo = 0;
        a.seg_cnt = 1;
        tm.before();
        e = kda::launch_chunk(a, st);
        tm.after();
        if (e != hipSuccess) return hip_fail(e, "chunk kernel launch");
        return KDA_OK;
    }
    float* ws = reinterpret_cast<float*>(workspace);
    const size_t per = (size_t)B * H * r.n_seg;
    float* s_loc = ws;
    float* m_tr = s_loc + per * dk * dv;
    float* starts = m_tr + per * dk * dk;
    const int2* seq_table = nullptr;
    if (r.packed_seg) {
        // packed sequences: the segment tables, built on the device from cu_seqlens
        char* tab = reinterpret_cast<char*>(workspace) + align256(per * (2 * (size_t)dk * dv + (size_t)dk * dk) * 4);
        kda::SegTableArgs t{cu, T, r.seg_len, r.n_seqs, r.n_seg, reinterpret_cast<int4*>(tab),
                            reinterpret_cast<int2*>(tab + align256((size_t)r.n_seg * 16))};
        tm.before();
        e = kda::launch_seg_table(t, st);
        tm.after();
        if (e != hipSuccess) return hip_fail(e, "segment table launch");
        a.seg_table = t.seg_table;
        a.cu_seqlens = nullptr;
        a.B = 1;
        seq_table = t.seq_table;
    }
    if (r.seg0_len > 0) {
        // lead form: segment 0 (from S0, in pass-2 form, its final state into starts[.., 1])
        // in one launch with pass 1 over segments 1 .. P-2; the scan from segment 1; pass 2
        // over segments 1 .. P-1
        kda::ChunkArgs a0 = a, a1 = a;
        a0.mode = 0;
        a0.s0 = S0;
        a0.starts = starts;
        a0.seg_lo = 0;
        a0.seg_cnt = 1;
        a1.mode = 1;
        a1.s_loc = s_loc;
        a1.m_tr = m_tr;
        a1.seg_lo = 1;
        a1.seg_cnt = r.n_seg - 2;
        tm.before();
        e = kda::launch_chunk_lead(a0, a1, st);
        tm.after();
        if (e != hipSuccess) return hip_fail(e, "lead launch");
        if (r.n_seg > 2) {
            kda::ScanArgs sc{S0, s_loc, m_tr, starts, B, H, dk, dv, r.n_seg, 1, nullptr};
            tm.before();
            e = kda::launch_scan(sc, st);
            tm.after();
            if (e != hipSuccess) return hip_fail(e, "segment scan launch");
        }
        a.mode = 0;
        a.s0 = nullptr;
        a.starts = starts;
        a.seg_lo = 1;
        a.seg_cnt = r.n_seg - 1;
        tm.before();
        e = kda::launch_chunk(a, st);
        tm.after();
        if (e != hipSuccess) return hip_fail(e, "segment pass-2 launch");
        return KDA_OK;
    }
    // pass 1: segment pairs (packed sequences: every slot; the kernel skips last segments)
    a.mode = 1;
    a.s_loc = s_loc;
    a.m_tr = m_tr;
    a.seg_lo = 0;
    a.seg_cnt = r.packed_seg ? r.n_seg : r.n_seg - 1;
    tm.before();
    e = kda::launch_chunk(a, st);
    tm.after();
    if (e != hipSuccess) return hip_fail(e, "segment pass-1 launch");
    // prefix scan over the pairs
    kda::ScanArgs sc{S0, s_loc, m_tr, starts, r.packed_seg ? (int64_t)r.n_seqs : B, H, dk, dv, r.n_seg, 0, seq_table};
    tm.before();
    e = kda::launch_scan(sc, st);
    tm.after();
    if (e != hipSuccess) return hip_fail(e, "segment scan launch");
    // pass 2: every segment from its true start state
    a.mode = 0;
    a.s0 = nullptr;
    a.starts = starts;
    a.seg_lo = 0;
    a.seg_cnt = r.n_seg;
    tm.before();
    e = kda::launch_chunk(a, st);
    tm.after();
    if (e != hipSuccess) return hip_fail(e, "segment pass-2 launch");
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status_t kda_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                           const float* beta, const float* S0, void* o, float* S_T, int64_t B,
                           int64_t T, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                           kda_dtype_t dt, const kda_plan_t* plan, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, S0, o, S_T, B, T, H, dk, dv, chunk, dt, plan, workspace,
                          workspace_bytes, stream, false);
}

kda_status_t kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const float* log_alpha,
                                   const float* beta, const float* S0, void* o, float* S_T, int64_t B,
                                   int64_t T, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                                   kda_dtype_t dt, const kda_plan_t* plan, void* stream) {
    return chunk_fwd_impl(q, k, v, log_alpha, beta, S0, o, S_T, B, T, H, dk, dv, chunk, dt, plan, nullptr, 0,
                          stream, true);
}

}  // extern "C"

namespace {

// Shared validation of the decode family: n_tok tokens per sequence; `state_out` says whether
// the call writes the state (then it must overlap no input), `o` may be null (commit).
kda_status_t decode_call(int mode, float* state, const void* q, const void* k, const void* v,
                         const float* log_alpha, const float* beta, void* o, const int32_t* n_accept,
                         int64_t N, int32_t n_tok, int32_t H, int32_t dk, int32_t dv, kda_dtype_t dt,
                         uint32_t flags, void* stream) {
    if (N < 1 || H < 1 || n_tok < 1)
        return fail(KDA_ERR_SHAPE, "need N >= 1, H >= 1, n_draft >= 1 (got N=%lld H=%d n=%d)", (long long)N, H, n_tok);
    if (dt != KDA_DTYPE_F32 && dt != KDA_DTYPE_BF16) return fail(KDA_ERR_DTYPE, "unknown dtype %d", (int)dt);
    if (!dim_ok(dk) || !dim_ok(dv)) return fail(KDA_ERR_UNSUPPORTED, "dk, dv must be 16, 32, 64 or 128 (got %d, %d)", dk, dv);
    if (flags & ~kAllFlags) return fail(KDA_ERR_UNSUPPORTED, "unknown input flags 0x%x", flags);
    if (N * (int64_t)H * n_tok > 0x7fffffff) return fail(KDA_ERR_SHAPE, "N * n_draft * H too large");
    const bool want_o = mode != kda::DECODE_COMMIT;
    if (!state || !q || !k || !v || !log_alpha || !beta || (want_o && !o) || (!want_o && !n_accept))
        return fail(KDA_ERR_NULL, "all pointers are required");
    const void* ptrs[] = {state, q, k, v, log_alpha, beta, o};
    for (const void* p : ptrs)
        if (p && !aligned(p)) return fail(KDA_ERR_ALIGN, "pointer %p is not 16-byte aligned", p);
    if (n_accept && reinterpret_cast<uintptr_t>(n_accept) % 4 != 0) return fail(KDA_ERR_ALIGN, "n_accept is not 4-byte aligned");
    const size_t es = dt == KDA_DTYPE_BF16 ? 2 : 4;
    const size_t nh = (size_t)N * H, nth = nh * n_tok;
    struct Span { const void* p; size_t n; const char* name; } ins[] = {
        {state, nh * dk * dv * 4, "state"}, {q, nth * dk * es, "q"}, {k, nth * dk * es, "k"}, {v, nth * dv * es, "v"},
        {log_alpha, nth * dk * 4, "log_alpha"}, {beta, nth * 4, "beta"}, {n_accept, n_accept ? (size_t)N * 4 : 0, "n_accept"}};
    if (want_o)
        for (const Span& in : ins)
            if (overlaps(o, nth * dv * es, in.p, in.n)) return fail(KDA_ERR_ALIAS, "o overlaps %s", in.name);
    if (mode != kda::DECODE_VERIFY)
        for (int i = 1; i < 7; ++i)
            if (overlaps(state, ins[0].n, ins[i].p, ins[i].n)) return fail(KDA_ERR_ALIAS, "state overlaps %s", ins[i].name);
    kda::DecodeArgs a{};
    a.state = state; a.q = q; a.k = k; a.v = v; a.log_alpha = log_alpha; a.beta = beta;
    a.o = want_o ? o : nullptr;
    a.n_accept = n_accept;
    a.N = N; a.n_tok = n_tok; a.H = H; a.dk = dk; a.dv = dv;
    a.mode = mode; a.flags = flags; a.bf16 = dt == KDA_DTYPE_BF16;
    hipError_t e = kda::launch_decode(a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status_t kda_decode_step(float* state, const void* q, const void* k, const void* v,
                             const float* log_alpha, const float* beta, void* o, int64_t N,
                             int32_t H, int32_t dk, int32_t dv, kda_dtype_t dt, uint32_t flags,
                             void* stream) {
    return decode_call(kda::DECODE_STEP, state, q, k, v, log_alpha, beta, o, nullptr, N, 1, H, dk, dv, dt,
                       flags, stream);
}

kda_status_t kda_decode_verify(const float* state, const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta, void* o, int64_t N,
                               int32_t n_draft, int32_t H, int32_t dk, int32_t dv, kda_dtype_t dt,
                               uint32_t flags, void* stream) {
    // the kernel of this mode never writes the state
    return decode_call(kda::DECODE_VERIFY, const_cast<float*>(state), q, k, v, log_alpha, beta, o, nullptr, N,
                       n_draft, H, dk, dv, dt, flags, stream);
}

kda_status_t kda_decode_commit(float* state, const void* q, const void* k, const void* v,
                               const float* log_alpha, const float* beta, const int32_t* n_accept,
                               int64_t N, int32_t n_draft, int32_t H, int32_t dk, int32_t dv,
                               kda_dtype_t dt, uint32_t flags, void* stream) {
    return decode_call(kda::DECODE_COMMIT, state, q, k, v, log_alpha, beta, nullptr, n_accept, N, n_draft, H,
                       dk, dv, dt, flags, stream);
}

}  // extern "C"
