"""The algorithmic work bench.py divides by, pinned to figures derived independently of it.

The roofline fractions the benchmark reports are algorithmic bytes (or flops) over measured
time, so a slip in those formulas would misreport every fraction.  The per-unit figures below
are worked out by hand from the operation's definition (the state recurrence and what a
single pass must read and write: q, k, v, o in bf16, a per-channel log-decay and beta in
float32, the float32 state once in and once out for decode) and written here as numbers,
not formulas.  The launch split of a segmented plan is
checked by conservation: every token is read in full by exactly one pass-2-form launch, and
pass 1 summarises exactly the tokens of the segments that have a successor.
"""
import bench
import kda_synth as ks


def test_prefill_per_token_head():
    # dk = dv = 128, chunk 64, bf16 operands
    assert bench.prefill_bytes_per_token_head(128, 128, 2) == 1540
    assert round(bench.prefill_flops_per_token_head(128, 128, 64)) == 132693
    # float32 operands: q, k, v, o 4 bytes each, the log-decay row and beta as before
    assert bench.prefill_bytes_per_token_head(16, 16, 4) == 4 * (16 + 16 + 16 + 16) + 4 * 16 + 4


def test_decode_and_speculative_bytes():
    # 256 sequences x 32 heads, a 128 x 128 float32 state read and written once per step
    assert bench.decode_bytes_per_step(256, 32, 128, 128, 2) == 1_086_357_504
    # verify of n drafts reads the state once; commit reads and writes it
    state = 128 * 128 * 4
    assert bench.verify_bytes(1, 4, 1, 128, 128, 2) == state + 4 * 1540
    assert bench.commit_bytes(1, 4, 1, 128, 128, 2) == 2 * state + 4 * (1540 - 2 * 128 * 2) + 4


def test_single_pass_bytes_of_the_long_context_workload():
    r = ks.WORKLOADS[3]
    assert (r.B, r.T, r.H, r.dk, r.dv) == (1, 1 << 20, 32, 128, 128)
    # 51.68 GB for one pass over 2^20 tokens x 32 heads
    assert r.B * r.T * r.H * bench.prefill_bytes_per_token_head(r.dk, r.dv, 2) == 51_673_825_280


class _Plan:
    def __init__(self, n_segments, seg0_len=0):
        self.n_segments, self.dv_block, self.seg0_len = n_segments, 128, seg0_len


def _split(r, plan):
    """Token bytes of the pass-2-form launches and of pass 1, from launch_bytes."""
    out = dict(bench.launch_bytes(r, plan, 2))
    full = bench.prefill_bytes_per_token_head(r.dk, r.dv, 2)
    summ = r.dk * 2 + r.dv * 2 + 4 * r.dk + 4          # pass 1 reads k, v, log_alpha, beta
    return out, full, summ


def test_lead_form_launches_conserve_tokens():
    r = ks.WORKLOADS[3]
    seg0, lc = 1488 * 64, 1862 * 64                      # the default plan: segment 0, then 8 of lc
    assert seg0 + 8 * lc == r.T
    out, full, summ = _split(r, _Plan(9, seg0))
    st = r.B * r.H * r.dk * r.dv * 4
    pair = r.B * r.H * (r.dk * r.dv + r.dk * r.dk) * 4
    lead = out["chunk_lead_kernel (segment 0 beside segment pass 1)"]
    pass2 = out["chunk_kernel (pass 2)"]
    # pass 2 reads every token after segment 0 in full, plus 8 start states in and S_T out
    assert pass2 == r.B * (r.T - seg0) * r.H * full + 8 * st + st
    # the lead launch: segment 0 in full (S0 is zero here: no start-state read), its end state
    # out, and pass 1 over segments 1..7 (not the last one), each summary pair written
    assert lead == r.B * seg0 * r.H * full + st + r.B * 7 * lc * r.H * summ + 7 * pair
    assert out["scan_kernel"] == 7 * pair + st + 7 * st


def test_equal_segments_conserve_tokens():
    r = ks.WORKLOADS[1]
    out, full, summ = _split(r, _Plan(16))
    st = r.B * r.H * r.dk * r.dv * 4
    pair = r.B * r.H * (r.dk * r.dv + r.dk * r.dk) * 4
    assert r.T == 16 * 256                               # 16 segments of 256 tokens
    assert out["chunk_kernel (segment pass 1)"] == r.B * 15 * 256 * r.H * summ + 15 * pair
    assert out["chunk_kernel (pass 2)"] == r.B * r.T * r.H * full + 16 * st + st
    s0 = st if r.s0_std > 0 else 0
    assert out["scan_kernel"] == 15 * pair + s0 + 16 * st
