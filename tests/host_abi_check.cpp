// Host-only check of the C ABI layer (kda_api.cpp), built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_abi_cpu.py.  The kernel launchers and the
// workspace lookup are replaced by stubs that record what they were asked to do, so every
// argument path runs on the CPU: rejected calls must return the documented code and launch
// nothing; accepted calls must launch the documented sequence with the resolved plan.  Also
// checks the kernels' 32-bit per-lane offset formula (kda_internal.h) at the ABI's limits.
// Fake device addresses are never dereferenced.
//
// Prints one line per failed check and exits 1 if any failed, 0 otherwise.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "kda.h"
#include "kda_internal.h"

// ------------------------------------------------------------------ stubs of the device side
namespace {
struct Launch {
    std::string what;
    int mode;
    int64_t B, T;
    int32_t n_seg;
    int64_t seg_len;
    int32_t dv_block;
    const void* ws;
    int32_t seg_lo = 0, seg_cnt = 0;   // chunk launches: the segments covered; scan: first in seg_lo
    int64_t seg0_len = 0;
    int32_t seg_cnt1 = 0;              // lead launch: pass-1 segments beside segment 0
};
std::vector<Launch> g_launches;
unsigned char g_scratch_stub[64];
}  // namespace

namespace kda {
hipError_t launch_chunk(const ChunkArgs& a, hipStream_t) {
    g_launches.push_back({a.mode == 1 ? "pass1" : "chunk", a.mode, a.B, a.T, a.n_seg, a.seg_len, a.dv_block,
                          a.s_loc, a.seg_lo, a.seg_cnt, a.seg0_len});
    return hipSuccess;
}
hipError_t launch_chunk_lead(const ChunkArgs& a0, const ChunkArgs& a1, hipStream_t) {
    // a0 runs segment 0 in mode 0, a1 pass 1 (mode 1) over the segments after it
    const bool ok = a0.mode == 0 && a1.mode == 1 && a0.seg_lo == 0 && a0.seg_cnt == 1 && a1.seg_lo == 1 &&
                    a0.starts != nullptr && a1.s_loc != nullptr && a1.m_tr != nullptr &&
                    a0.seg0_len == a1.seg0_len && a0.seg_len == a1.seg_len && a0.n_seg == a1.n_seg;
    g_launches.push_back({ok ? "lead" : "lead-bad-args", 0, a0.B, a0.T, a0.n_seg, a0.seg_len, a0.dv_block,
                          a1.s_loc, a0.seg_lo, a0.seg_cnt, a0.seg0_len, a1.seg_cnt});
    return hipSuccess;
}
hipError_t launch_scan(const ScanArgs& a, hipStream_t) {
    g_launches.push_back({"scan", -1, a.B, 0, a.n_seg, 0, 0, a.s_loc, a.first});
    return hipSuccess;
}
hipError_t launch_decode(const DecodeArgs& a, hipStream_t) {
    g_launches.push_back({"decode", a.mode, a.N, a.n_tok, 0, 0, 0, nullptr});
    return hipSuccess;
}
hipError_t launch_seg_table(const SegTableArgs& a, hipStream_t) {
    g_launches.push_back({"segtable", -1, a.n_seqs, a.T, a.n_slots, a.seg_len, 0, a.seg_table});
    return hipSuccess;
}
hipError_t scratch_address(void** out) {
    *out = g_scratch_stub;
    return hipSuccess;
}
}  // namespace kda

// ------------------------------------------------------------------ checks
namespace {
int g_fail = 0;
#define CHECK(cond, ...)                                                  \
    do {                                                                  \
        if (!(cond)) {                                                    \
            ++g_fail;                                                     \
            std::printf("FAIL %s:%d: ", __FILE__, __LINE__);              \
            std::printf(__VA_ARGS__);                                     \
            std::printf("  [%s]\n", #cond);                               \
        }                                                                 \
    } while (0)

// fake device addresses: 16-byte aligned, 2^40 bytes apart, never dereferenced
void* A(int i) { return reinterpret_cast<void*>((uintptr_t)(i + 1) << 40); }
template <typename T> T* P(int i, size_t byte_off = 0) {
    return reinterpret_cast<T*>(reinterpret_cast<char*>(A(i)) + byte_off);
}

struct Call {
    const void *q = A(0), *k = A(1), *v = A(2);
    const float *la = P<float>(3), *beta = P<float>(4), *S0 = nullptr;
    void* o = A(6);
    float* S_T = P<float>(7);
    int64_t B = 1, T = 64;
    int32_t H = 2, dk = 16, dv = 16, chunk = 16;
    kda_dtype_t dt = KDA_DTYPE_F32;
    kda_plan_t plan{1, 0, nullptr, 0, nullptr, 0, nullptr, 0, 0};   // one pass unless a case says otherwise
    bool use_plan = true;
    void* ws = nullptr;
    size_t wsb = 0;
    kda_status_t run(bool noalloc = false) const {
        const kda_plan_t* p = use_plan ? &plan : nullptr;
        if (noalloc) return kda_chunk_fwd_noalloc(q, k, v, la, beta, S0, o, S_T, B, T, H, dk, dv, chunk, dt, p, nullptr);
        return kda_chunk_fwd(q, k, v, la, beta, S0, o, S_T, B, T, H, dk, dv, chunk, dt, p, ws, wsb, nullptr);
    }
};

void expect_reject(const Call& c, kda_status_t code, const char* what, bool noalloc = false) {
    g_launches.clear();
    const kda_status_t s = c.run(noalloc);
    CHECK(s == code, "%s: got %d, expected %d (%s)", what, (int)s, (int)code, kda_last_error());
    CHECK(g_launches.empty(), "%s: a rejected call launched %zu kernels", what, g_launches.size());
    CHECK(std::strlen(kda_last_error()) > 0, "%s: no message", what);
}

void chunk_errors() {
    Call c;
    { Call x = c; x.q = nullptr; expect_reject(x, KDA_ERR_NULL, "q null"); }
    { Call x = c; x.S_T = nullptr; expect_reject(x, KDA_ERR_NULL, "S_T null"); }
    { Call x = c; x.B = 0; expect_reject(x, KDA_ERR_SHAPE, "B = 0"); }
    { Call x = c; x.T = -1; expect_reject(x, KDA_ERR_SHAPE, "T < 0"); }
    { Call x = c; x.dt = (kda_dtype_t)7; expect_reject(x, KDA_ERR_DTYPE, "dtype"); }
    { Call x = c; x.dk = 24; expect_reject(x, KDA_ERR_UNSUPPORTED, "dk = 24"); }
    { Call x = c; x.chunk = 128; expect_reject(x, KDA_ERR_UNSUPPORTED, "chunk = 128"); }
    { Call x = c; x.dk = 128; x.chunk = 64; expect_reject(x, KDA_ERR_UNSUPPORTED, "f32 chunk*dk"); }
    { Call x = c; x.H = 1 << 17; x.dk = 128; x.T = 1; x.chunk = 16; x.dt = KDA_DTYPE_BF16;
      expect_reject(x, KDA_ERR_UNSUPPORTED, "H * dk = 2^24"); }
    { Call x = c; x.q = P<char>(0, 4); expect_reject(x, KDA_ERR_ALIGN, "q misaligned"); }
    { Call x = c; x.o = A(0); expect_reject(x, KDA_ERR_ALIAS, "o aliases q"); }
    { Call x = c; x.S_T = P<float>(1); expect_reject(x, KDA_ERR_ALIAS, "S_T aliases k"); }
    { Call x = c; x.S0 = P<float>(7, 16); expect_reject(x, KDA_ERR_ALIAS, "S0 partially overlaps S_T"); }
    { Call x = c; x.plan.dv_block = 24; expect_reject(x, KDA_ERR_UNSUPPORTED, "dv_block 24"); }
    { Call x = c; x.plan.n_segments = -1; expect_reject(x, KDA_ERR_UNSUPPORTED, "n_segments < 0"); }
    { Call x = c; x.plan.flags = 4; expect_reject(x, KDA_ERR_UNSUPPORTED, "unknown flag"); }
    { Call x = c; x.plan.state_ckpt = P<float>(9); x.plan.ckpt_stride = 24;
      expect_reject(x, KDA_ERR_UNSUPPORTED, "ckpt stride"); }
    { Call x = c; x.plan.state_ckpt = P<float>(6); x.plan.ckpt_stride = 32;
      expect_reject(x, KDA_ERR_ALIAS, "ckpt aliases o"); }
    { Call x = c; x.plan.cu_seqlens = P<int32_t>(10); x.plan.n_seqs = 3; x.B = 2;
      expect_reject(x, KDA_ERR_SHAPE, "packed with B = 2"); }
    { Call x = c; x.plan.cu_seqlens = P<int32_t>(10, 2); x.plan.n_seqs = 3;
      expect_reject(x, KDA_ERR_ALIGN, "cu_seqlens misaligned"); }
    { Call x = c; x.plan.n_launch_events = -1; x.plan.launch_events = reinterpret_cast<void* const*>(A(11));
      expect_reject(x, KDA_ERR_UNSUPPORTED, "negative event count"); }
    // segments without a workspace, or with one too small / overlapping an input
    Call s;
    s.T = 256; s.dk = s.dv = 32; s.dt = KDA_DTYPE_BF16; s.plan.n_segments = 4; s.plan.dv_block = 32;
    expect_reject(s, KDA_ERR_WORKSPACE, "segments, no workspace");
    { Call x = s; x.ws = A(8); x.wsb = 100; expect_reject(x, KDA_ERR_WORKSPACE, "workspace too small"); }
    { Call x = s; x.ws = A(2); x.wsb = 1 << 20; expect_reject(x, KDA_ERR_ALIAS, "workspace aliases v"); }
    // kda_chunk_fwd_noalloc: a plan beyond the library's workspace
    { Call x; x.T = 1 << 16; x.H = 64; x.dk = x.dv = 128; x.chunk = 64; x.dt = KDA_DTYPE_BF16;
      x.plan.n_segments = 16; x.plan.dv_block = 128;
      expect_reject(x, KDA_ERR_WORKSPACE, "noalloc beyond its workspace", true); }
}

void chunk_launches() {
    // one pass
    Call c;
    g_launches.clear();
    CHECK(c.run() == KDA_OK, "one pass: %s", kda_last_error());
    CHECK(g_launches.size() == 1 && g_launches[0].mode == 0 && g_launches[0].n_seg == 1, "one pass launches");
    // the default plan of the B1 T4096 H16 prefill: 16 segments, three launches
    Call d;
    d.T = 4096; d.H = 16; d.dk = d.dv = 128; d.chunk = 64; d.dt = KDA_DTYPE_BF16; d.use_plan = false;
    size_t need = 0;
    CHECK(kda_chunk_fwd_workspace_bytes(1, 4096, 16, 128, 128, 64, KDA_DTYPE_BF16, nullptr, &need) == KDA_OK, "ws query");
    CHECK(need == (size_t)16 * 16 * 3 * 128 * 128 * 4, "workspace of the default plan: %zu", need);
    d.ws = A(8);
    d.wsb = need;
    g_launches.clear();
    CHECK(d.run() == KDA_OK, "segmented: %s", kda_last_error());
    CHECK(g_launches.size() == 3, "segmented: %zu launches", g_launches.size());
    if (g_launches.size() == 3) {
        CHECK(g_launches[0].what == "pass1" && g_launches[1].what == "scan" && g_launches[2].what == "chunk",
              "launch order");
        CHECK(g_launches[0].n_seg == 16 && g_launches[0].seg_len == 256, "plan %d x %lld", g_launches[0].n_seg,
              (long long)g_launches[0].seg_len);
        CHECK(g_launches[0].ws == A(8), "the caller's workspace is used");
        // equal segments: pass 1 over segments 0 .. 14, the scan from S0, pass 2 over all 16
        CHECK(g_launches[0].seg_lo == 0 && g_launches[0].seg_cnt == 15 && g_launches[0].seg0_len == 0, "pass-1 range");
        CHECK(g_launches[1].seg_lo == 0, "scan from S0");
        CHECK(g_launches[2].seg_lo == 0 && g_launches[2].seg_cnt == 16, "pass-2 range");
    }
    // the same through kda_chunk_fwd_noalloc: the library's workspace
    g_launches.clear();
    CHECK(d.run(true) == KDA_OK, "noalloc: %s", kda_last_error());
    CHECK(g_launches.size() == 3 && g_launches[0].ws == g_scratch_stub, "noalloc uses the library workspace");
    // the 1M-token workload's default plan: the lead form of 9 segments
    kda_plan_t p{};
    CHECK(kda_chunk_fwd_default_plan(1, 1 << 20, 32, 128, 128, 64, KDA_DTYPE_BF16, &p) == KDA_OK, "plan query");
    // 8 equal segments would fill the 256 CUs in pass 2 (cost 2048 x 1.8 = 3686.4 pass-2 chunks);
    // the lead form with l = 1862 (l = floor(16384 / 8.8) = 1861 costs 1496 + 1861 = 3357; 1862
    // costs max(1488, 1489.6) + 1862 = 3351.6) adds segment 0 of 1488 chunks beside pass 1
    CHECK(p.n_segments == 9 && p.dv_block == 128 && p.seg0_len == 1488 * 64, "1M plan %d / %d / %lld",
          p.n_segments, p.dv_block, (long long)p.seg0_len);
    // 4 units (B2 H2): 64 equal segments of 20 chunks cost 36; at 1,280 chunks the lead form's
    // whole segments leave segment 0 either 64 chunks long (l = 19) or empty (l = 20), so the
    // default keeps equal segments; at 1,230 chunks l = 19 leaves 14 (cost 34.2) and it leads
    {
        kda_plan_t q{};
        CHECK(kda_chunk_fwd_default_plan(2, 81920, 2, 64, 64, 64, KDA_DTYPE_BF16, &q) == KDA_OK && q.n_segments == 64 &&
                  q.seg0_len == 0, "B2 T81920 H2 plan %d / %lld", q.n_segments, (long long)q.seg0_len);
        CHECK(kda_chunk_fwd_default_plan(2, 78720, 2, 64, 64, 64, KDA_DTYPE_BF16, &q) == KDA_OK && q.n_segments == 65 &&
                  q.seg0_len == 14 * 64, "B2 T78720 H2 plan %d / %lld", q.n_segments, (long long)q.seg0_len);
        CHECK(kda_chunk_fwd_default_plan(1, 4096, 16, 128, 128, 64, KDA_DTYPE_BF16, &q) == KDA_OK && q.n_segments == 16 &&
                  q.seg0_len == 0, "B1 T4096 H16 plan %d / %lld", q.n_segments, (long long)q.seg0_len);
    }
    {
        Call m;
        m.T = 1 << 20; m.H = 32; m.dk = m.dv = 128; m.chunk = 64; m.dt = KDA_DTYPE_BF16; m.use_plan = false;
        m.S0 = P<float>(5);
        size_t need_m = 0;
        CHECK(kda_chunk_fwd_workspace_bytes(1, 1 << 20, 32, 128, 128, 64, KDA_DTYPE_BF16, nullptr, &need_m) == KDA_OK,
              "1M ws query");
        CHECK(need_m == (size_t)32 * 9 * 3 * 128 * 128 * 4, "1M workspace %zu", need_m);
        m.ws = A(8);
        m.wsb = need_m;
        g_launches.clear();
        CHECK(m.run() == KDA_OK, "1M lead plan: %s", kda_last_error());
        CHECK(g_launches.size() == 3, "1M lead plan: %zu launches", g_launches.size());
        if (g_launches.size() == 3) {
            CHECK(g_launches[0].what == "lead" && g_launches[0].seg_cnt1 == 7 && g_launches[0].seg0_len == 1488 * 64 &&
                      g_launches[0].seg_len == 1862 * 64 && g_launches[0].n_seg == 9,
                  "lead launch: %s pass-1 segments %d seg0 %lld seg_len %lld", g_launches[0].what.c_str(),
                  g_launches[0].seg_cnt1, (long long)g_launches[0].seg0_len, (long long)g_launches[0].seg_len);
            CHECK(g_launches[1].what == "scan" && g_launches[1].seg_lo == 1, "scan from segment 1");
            CHECK(g_launches[2].what == "chunk" && g_launches[2].seg_lo == 1 && g_launches[2].seg_cnt == 8,
                  "pass 2 over segments 1 .. 8");
        }
        // re-resolving the default plan explicitly gives the same execution
        Call e = m;
        e.use_plan = true;
        e.plan = p;
        g_launches.clear();
        CHECK(e.run() == KDA_OK && g_launches.size() == 3 && g_launches[0].seg_len == 1862 * 64 &&
                  g_launches[0].seg0_len == 1488 * 64,
              "explicit copy of the default plan");
        // the lead form's own checks
        { Call x = e; x.plan.seg0_len = 100; expect_reject(x, KDA_ERR_UNSUPPORTED, "seg0_len not a multiple of chunk"); }
        { Call x = e; x.plan.seg0_len = (int64_t)1 << 20; expect_reject(x, KDA_ERR_UNSUPPORTED, "seg0_len = T"); }
        { Call x = e; x.plan.seg0_len = -64; expect_reject(x, KDA_ERR_UNSUPPORTED, "seg0_len < 0"); }
        { Call x = e; x.plan.n_segments = 1; expect_reject(x, KDA_ERR_UNSUPPORTED, "seg0_len with one segment"); }
        // two segments: segment 0 alone in the lead launch, no scan, pass 2 over segment 1
        Call two = e;
        two.plan.n_segments = 2;
        two.plan.seg0_len = 4096;
        g_launches.clear();
        CHECK(two.run() == KDA_OK, "two-segment lead plan: %s", kda_last_error());
        CHECK(g_launches.size() == 2 && g_launches[0].what == "lead" && g_launches[0].seg_cnt1 == 0 &&
                  g_launches[1].what == "chunk" && g_launches[1].seg_lo == 1 && g_launches[1].seg_cnt == 1 &&
                  g_launches[1].seg_len == ((1 << 20) - 4096),
              "two-segment lead launches (%zu)", g_launches.size());
    }
    // packed sequences with segments: segment table, pass 1, scan, pass 2; segments of
    // ceil(T / n_segments) tokens rounded up to whole chunks; ceil(T / seg_len) + n_seqs slots
    Call pk;
    pk.T = 70000; pk.H = 4; pk.dk = pk.dv = 128; pk.chunk = 64; pk.dt = KDA_DTYPE_BF16;
    pk.plan.n_segments = 0;
    pk.plan.cu_seqlens = P<int32_t>(10);
    pk.plan.n_seqs = 5;
    pk.S0 = P<float>(5);
    size_t need_pk = 0;
    CHECK(kda_chunk_fwd_workspace_bytes(1, 70000, 4, 128, 128, 64, KDA_DTYPE_BF16, &pk.plan, &need_pk) == KDA_OK,
          "packed ws query: %s", kda_last_error());
    expect_reject(pk, KDA_ERR_WORKSPACE, "packed segments without a workspace");
    { Call x = pk; x.plan.seg0_len = 64; expect_reject(x, KDA_ERR_UNSUPPORTED, "seg0_len with packed sequences"); }
    pk.ws = A(8);
    pk.wsb = need_pk;
    g_launches.clear();
    CHECK(pk.run() == KDA_OK, "packed segments: %s", kda_last_error());
    CHECK(g_launches.size() == 4, "packed segments: %zu launches", g_launches.size());
    if (g_launches.size() == 4) {
        // 64 target segments over 70,000 tokens: 1094 -> 18 chunks = 1152 tokens; 61 + 5 slots
        CHECK(g_launches[0].what == "segtable" && g_launches[0].seg_len == 1152 && g_launches[0].n_seg == 66,
              "table: seg_len %lld slots %d", (long long)g_launches[0].seg_len, g_launches[0].n_seg);
        CHECK(g_launches[1].what == "pass1" && g_launches[1].n_seg == 66 && g_launches[1].B == 1, "packed pass 1");
        CHECK(g_launches[2].what == "scan" && g_launches[2].B == 5 && g_launches[2].n_seg == 66, "packed scan");
        CHECK(g_launches[3].what == "chunk" && g_launches[3].mode == 0, "packed pass 2");
        CHECK(need_pk == 256 * ((66u * 4 * 3 * 128 * 128 * 4 + 255) / 256) + 256 * ((66 * 16 + 255) / 256) + 5 * 8,
              "packed workspace %zu", need_pk);
    }
    // packed sequences that already cover the compute units: one pass
    Call pk1 = pk;
    pk1.plan.n_seqs = 64;
    pk1.ws = nullptr;
    pk1.wsb = 0;
    g_launches.clear();
    CHECK(pk1.run() == KDA_OK && g_launches.size() == 1, "64 packed sequences x 4 heads: one pass");
    // T = 0: one launch that copies S0 into S_T
    Call z;
    z.T = 0;
    z.q = z.k = z.v = z.o = nullptr;
    z.la = z.beta = nullptr;
    g_launches.clear();
    CHECK(z.run() == KDA_OK, "T = 0: %s", kda_last_error());
}

void decode_errors_and_launches() {
    g_launches.clear();
    kda_status_t s = kda_decode_step(P<float>(0), A(1), A(2), A(3), P<float>(4), P<float>(5), A(6), 4, 2, 16, 16,
                                     KDA_DTYPE_BF16, 0, nullptr);
    CHECK(s == KDA_OK && g_launches.size() == 1, "decode step");
    g_launches.clear();
    s = kda_decode_step(P<float>(0), A(1), A(2), A(3), P<float>(4), P<float>(5), A(0), 4, 2, 16, 16, KDA_DTYPE_BF16,
                        0, nullptr);
    CHECK(s == KDA_ERR_ALIAS && g_launches.empty(), "decode o aliases state");
    s = kda_decode_verify(P<float>(0), A(1), A(2), A(3), P<float>(4), P<float>(5), P<char>(1, 32), 4, 3, 2, 16, 16,
                          KDA_DTYPE_BF16, 0, nullptr);
    CHECK(s == KDA_ERR_ALIAS && g_launches.empty(), "verify o overlaps q");
    s = kda_decode_commit(P<float>(0), A(1), A(2), A(3), P<float>(4), P<float>(5), P<int32_t>(7, 2), 4, 3, 2, 16,
                          16, KDA_DTYPE_BF16, 0, nullptr);
    CHECK(s == KDA_ERR_ALIGN && g_launches.empty(), "commit n_accept misaligned");
    s = kda_decode_commit(P<float>(0), A(1), A(2), A(3), P<float>(4), P<float>(5), nullptr, 4, 3, 2, 16, 16,
                          KDA_DTYPE_BF16, 0, nullptr);
    CHECK(s == KDA_ERR_NULL && g_launches.empty(), "commit without n_accept");
}

// The kernels' per-lane offsets: (tok * stride + col) * esize in 32 bits, tok < 64.
void offsets() {
    // largest stride the ABI accepts for each dk (H * max(dk, dv) < 2^24, 16-byte multiples)
    for (int dk : {16, 32, 64, 128}) {
        const int32_t H = (int32_t)(((1 << 24) - 1) / dk);
        const unsigned stride = (unsigned)H * (unsigned)dk;
        CHECK(stride < (1u << 24), "stride");
        Call x;
        x.H = H; x.dk = x.dv = dk; x.T = 1; x.chunk = 16; x.dt = KDA_DTYPE_BF16;
        g_launches.clear();
        CHECK(x.run() == KDA_OK, "the largest accepted H for dk=%d is rejected: %s", dk, kda_last_error());
        for (unsigned esize : {2u, 4u})
            for (unsigned tok = 0; tok < 64; ++tok)
                for (unsigned col : {0u, (unsigned)dk - 4u, (unsigned)dk - 1u}) {
                    const uint64_t exact = ((uint64_t)tok * stride + col) * esize;
                    const uint64_t got = (uint64_t)(kda::tok_elem_off(tok, stride, col) * esize);
                    CHECK(exact < (1ull << 32) && got == exact, "dk=%d H=%d tok=%u col=%u esize=%u: %llu vs %llu", dk, H,
                          tok, col, esize, (unsigned long long)got, (unsigned long long)exact);
                }
    }
    // the 1M-token workload (H = 32, dk = dv = 128): the largest per-lane offsets
    for (unsigned esize : {2u, 4u}) {
        const uint64_t exact = (63ull * 4096 + 127) * esize;
        CHECK((uint64_t)(kda::tok_elem_off(63, 4096, 127) * esize) == exact, "1M workload offset");
    }
    // one past the bound would wrap: the ABI limit is where the formula stops being exact
    const unsigned over = 1u << 24;
    CHECK(kda::tok_elem_off(1, over, 0) != over, "a 2^24 stride must not fit the 24-bit multiply");
}
}  // namespace

// "plans" mode: one problem per stdin line, "B T H dk dv chunk dtype".  For each, the launches
// kda_chunk_fwd makes under the default plan, then under an explicit copy of the plan that
// kda_chunk_fwd_default_plan returns, one output line per problem:
//   status workspace n_segments dv_block seg0_len | launches of the default | launches of the copy
// with a launch written what:mode:seg_lo:seg_cnt:seg_cnt1:n_seg:seg_len:seg0_len:dv_block:B
// (scan: seg_lo is the first segment it starts from).
void print_launches() {
    for (const Launch& L : g_launches)
        std::printf(" %s:%d:%d:%d:%d:%d:%lld:%lld:%d:%lld", L.what.c_str(), L.mode, L.seg_lo, L.seg_cnt, L.seg_cnt1,
                    L.n_seg, (long long)L.seg_len, (long long)L.seg0_len, L.dv_block, (long long)L.B);
}

int plans() {
    char line[256];
    while (std::fgets(line, sizeof line, stdin)) {
        long long B = 0, T = 0;
        int H = 0, dk = 0, dv = 0, chunk = 0, dt = 0;
        if (std::sscanf(line, "%lld %lld %d %d %d %d %d", &B, &T, &H, &dk, &dv, &chunk, &dt) != 7) continue;
        Call c;
        c.B = B; c.T = T; c.H = H; c.dk = dk; c.dv = dv; c.chunk = chunk; c.dt = (kda_dtype_t)dt;
        c.use_plan = false;
        size_t need = 0;
        kda_plan_t p{};
        kda_status_t s = kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, c.dt, nullptr, &need);
        if (s == KDA_OK) s = kda_chunk_fwd_default_plan(B, T, H, dk, dv, chunk, c.dt, &p);
        c.ws = need ? A(8) : nullptr;
        c.wsb = need;
        g_launches.clear();
        if (s == KDA_OK) s = c.run();
        std::printf("%d %zu %d %d %lld |", (int)s, need, p.n_segments, p.dv_block, (long long)p.seg0_len);
        print_launches();
        Call e = c;
        e.use_plan = true;
        e.plan = p;
        g_launches.clear();
        if (s == KDA_OK) s = e.run();
        std::printf(" |");
        print_launches();
        std::printf(" %d\n", (int)s);
    }
    return 0;
}

int main(int argc, char** argv) {
    if (argc > 1 && std::strcmp(argv[1], "plans") == 0) return plans();
    if (argc > 1 && std::strcmp(argv[1], "trace") == 0) {
        // one segmented call; the test reads the KDA_TRACE line from stderr
        Call d;
        d.T = 4096; d.H = 16; d.dk = d.dv = 128; d.chunk = 64; d.dt = KDA_DTYPE_BF16; d.use_plan = false;
        return d.run(true) == KDA_OK ? 0 : 1;
    }
    chunk_errors();
    chunk_launches();
    decode_errors_and_launches();
    offsets();
    std::printf("%s: %d failed checks\n", g_fail ? "FAIL" : "ok", g_fail);
    return g_fail ? 1 : 0;
}
