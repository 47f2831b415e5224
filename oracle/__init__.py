"""CPU oracle (float64 numpy) for the KDA hot path -- test infrastructure only.

Imported by tests/, __graft_entry__.smoke() and the benchmark's cpu_baseline
leg; never by the library's product path.
"""
from .kda import *  # noqa: F401,F403
from .kda import (LOG_ALPHA_FLOOR, SUBTILE, QK_NORM_EPS, floor_log_alpha, gate_from_logits, l2_normalize,  # noqa: F401
                  kda_loop,
                  kda_decode_step, kda_decode_verify, kda_decode_commit,
                  kda_bruteforce, kda_chunked, gla_loop, gdn_loop, segment_transition,
                  segment_pairs, compose, segment_start_states, kda_segmented, rel_fro)
