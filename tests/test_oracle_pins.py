"""Pins for the CPU oracle: closed forms, independently written reductions,
exact rational arithmetic, brute force and invariants.

Every check here runs on the CPU (no GPU marker).  Shapes use dk != dv so a
transposed state (decay applied to value columns instead of key rows) fails.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import rel_fro

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd_inputs(seed, B=2, T=12, H=3, dk=5, dv=3, loga_lo=-5.0, beta_max=1.0, s0=True, unit_k=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    la = rng.uniform(loga_lo, 0.0, (B, T, H, dk))
    beta = rng.uniform(0.0, beta_max, (B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, la, beta, S0


# ---------------------------------------------------------------- P14 constants

def _golden_constants():
    vals = {}
    with open(os.path.join(GOLDEN, "floor_constants.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, val = line.split()[:2]
                vals[name] = float(val)
    return vals


def test_page_floor_constants():
    """The floor numbers printed on the page follow from log-alpha >= -5 and 16-token tiles."""
    import torch
    g = _golden_constants()
    floor, tile = oracle.LOG_ALPHA_FLOOR, oracle.SUBTILE
    assert round(100 * math.exp(floor), 2) == g["keep_per_step_percent"]
    assert tile == g["tile_tokens"]
    assert tile * floor == g["tile_log_decay_min"]
    recip = math.exp(-tile * floor)
    assert round(recip / 1e34, 1) * 1e34 == pytest.approx(g["reciprocal_bound"])
    bf16_max = float(torch.finfo(torch.bfloat16).max)
    assert round(bf16_max / 1e38, 1) * 1e38 == pytest.approx(g["bf16_max"])
    assert recip < bf16_max and recip < float(torch.finfo(torch.float32).max)
    # one tile more would not fit: e^(-5*32) overflows fp32 and bf16
    assert math.exp(-2 * tile * floor) > float(torch.finfo(torch.float32).max)


# ---------------------------------------------------------------- P7 brute force

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_loop_matches_bruteforce(seed):
    x = rnd_inputs(seed, T=7)
    o1, S1 = oracle.kda_loop(*x)
    o2, S2 = oracle.kda_bruteforce(*x)
    assert rel_fro(o1, o2) < 1e-12 and rel_fro(S1, S2) < 1e-12


def _frac_matmul(A, B):
    return [[sum(A[i][k] * B[k][j] for k in range(len(B))) for j in range(len(B[0]))]
            for i in range(len(A))]


def test_loop_matches_exact_rational():
    """Exact rational evaluation of the definition on a tiny case (dk=2, dv=3, T=3)."""
    F = Fraction
    alphas = [[F(1, 2), F(3, 4)], [F(1, 1), F(1, 3)], [F(2, 3), F(1, 2)]]
    betas = [F(1, 2), F(1, 1), F(1, 4)]
    ks = [[F(3, 5), F(4, 5)], [F(1, 1), F(0)], [F(-4, 5), F(3, 5)]]
    vs = [[F(1), F(-2), F(1, 2)], [F(3, 2), F(0), F(-1)], [F(-1, 3), F(2), F(1)]]
    qs = [[F(1, 2), F(-1)], [F(2), F(1, 3)], [F(-1, 4), F(1)]]
    S = [[F(1, 3), F(0), F(-1)], [F(1, 2), F(2), F(0)]]
    S0 = [row[:] for row in S]
    outs = []
    for t in range(3):
        Pm = [[(F(1) if i == j else F(0)) - betas[t] * ks[t][i] * ks[t][j] for j in range(2)] for i in range(2)]
        Dm = [[alphas[t][i] if i == j else F(0) for j in range(2)] for i in range(2)]
        S = _frac_matmul(_frac_matmul(Pm, Dm), S)
        S = [[S[i][j] + betas[t] * ks[t][i] * vs[t][j] for j in range(3)] for i in range(2)]
        outs.append([sum(S[i][j] * qs[t][i] for i in range(2)) for j in range(3)])
    f = lambda a: np.array(a, dtype=np.float64)  # noqa: E731
    la = np.log(f(alphas))
    o, S_T = oracle.kda_loop(f(qs)[None, :, None], f(ks)[None, :, None], f(vs)[None, :, None],
                             la[None, :, None], f(betas)[None, :, None], f(S0)[None, None])
    assert np.abs(o[0, :, 0] - f(outs)).max() < 1e-14
    assert np.abs(S_T[0, 0] - f(S)).max() < 1e-14


# ---------------------------------------------------------------- P1 beta = 0

def test_beta_zero_is_pure_decay():
    q, k, v, la, beta, S0 = rnd_inputs(3)
    beta = np.zeros_like(beta)
    o, S_T = oracle.kda_loop(q, k, v, la, beta, S0)
    G = np.cumsum(la, axis=1)                                  # [B,T,H,dk]
    o_ref = np.einsum("bhcj,bthc->bthj", S0, q * np.exp(G))
    S_ref = np.exp(G[:, -1])[..., None] * S0
    assert rel_fro(o, o_ref) < 1e-13 and rel_fro(S_T, S_ref) < 1e-13


# ---------------------------------------------------------------- P2 GLA limit

def test_small_beta_is_gla_limit():
    q, k, v, la, beta, _ = rnd_inputs(4, T=20)
    eps = 1e-7
    o, _ = oracle.kda_loop(q, k, v, la, np.full_like(beta, eps), None)
    o_gla = oracle.gla_loop(q, k, v, la, None)
    err = rel_fro(o / eps, o_gla)
    assert err < 1e-5
    # and the difference is first order in eps (a missing erase term would show as O(1))
    o2, _ = oracle.kda_loop(q, k, v, la, np.full_like(beta, 2 * eps), None)
    err2 = rel_fro(o2 / (2 * eps), o_gla)
    assert 1.5 < err2 / err < 2.5


# ---------------------------------------------------------------- the reductions' own definitions

def test_gla_loop_against_decayed_causal_sum():
    """gla_loop against its closed form, written as a double sum over position pairs with the
    decay as an explicit product of per-step factors (no cumulative sums of logs):
    o_t = sum_c q_tc [ (prod_{r<=t} a_rc) S0[c,:] + sum_{s<=t} (prod_{s<r<=t} a_rc) k_sc v_s ]."""
    q, k, v, la, _, S0 = rnd_inputs(21, B=1, T=9, H=2, dk=4, dv=3)
    a = np.exp(np.clip(la, -5.0, 0.0))
    B, T, H, dk = q.shape
    o_ref = np.zeros(v.shape)
    for h in range(H):
        for t in range(T):
            for c in range(dk):
                prod_all = np.prod(a[0, :t + 1, h, c])
                acc = prod_all * S0[0, h, c]
                for s in range(t + 1):
                    acc = acc + np.prod(a[0, s + 1:t + 1, h, c]) * k[0, s, h, c] * v[0, s, h]
                o_ref[0, t, h] += q[0, t, h, c] * acc
    o = oracle.gla_loop(q, k, v, la, S0)
    assert rel_fro(o, o_ref) < 1e-13


def test_gdn_loop_against_matrix_products():
    """gdn_loop against explicit dk x dk matrices: S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T
    with the products formed as np.outer / np.eye, and a hand-checked two-step case."""
    q, k, v, la, beta, S0 = rnd_inputs(22, B=1, T=6, H=1, dk=4, dv=2)
    la_h = la[..., 0]
    a = np.exp(np.clip(la_h, -5.0, 0.0))
    S = S0[0, 0].copy()
    o_ref = np.empty((6, 2))
    for t in range(6):
        P = a[0, t, 0] * (np.eye(4) - beta[0, t, 0] * np.outer(k[0, t, 0], k[0, t, 0]))
        S = P @ S + beta[0, t, 0] * np.outer(k[0, t, 0], v[0, t, 0])
        o_ref[t] = q[0, t, 0] @ S
    o, S_T = oracle.gdn_loop(q, k, v, la_h, beta, S0)
    assert rel_fro(o[0, :, 0], o_ref) < 1e-13 and rel_fro(S_T[0, 0], S) < 1e-13
    # dk = 1, dv = 1 by hand: a = 1/2, b = 1, k = 1: S1 = 0.5 (1 - 1) S0 + v1 = v1; S2 = 0.5 * 0 + v2
    one = np.ones((1, 2, 1, 1))
    o2, S2 = oracle.gdn_loop(one, one, np.array([3.0, -2.0]).reshape(1, 2, 1, 1),
                             np.full((1, 2, 1), np.log(0.5)), np.ones((1, 2, 1)), np.full((1, 1, 1, 1), 7.0))
    assert np.allclose(o2.ravel(), [3.0, -2.0], atol=1e-15) and np.allclose(S2.ravel(), [-2.0], atol=1e-15)


def test_rel_fro_is_normalised_by_the_reference():
    """Every parity claim uses rel_fro: pin it by hand.  ref = 3 e1 and x = ref + 4 e2 give
    ||x - ref|| / ||ref|| = 4 / 3 (normalising by ||x|| = 5 would give 4 / 5)."""
    ref = np.array([3.0, 0.0])
    x = ref + np.array([0.0, 4.0])
    assert rel_fro(x, ref) == pytest.approx(4.0 / 3.0, rel=1e-15)
    assert rel_fro(ref, x) == pytest.approx(4.0 / 5.0, rel=1e-15)      # the arguments are not symmetric
    assert rel_fro(ref, ref) == 0.0
    # over a whole tensor, not per row: rows [3, 0] and [0, 4] against [3, 4] and [0, 0]
    assert rel_fro(np.array([[3.0, 0.0], [0.0, 4.0]]), np.array([[3.0, 4.0], [0.0, 0.0]])) == \
        pytest.approx(math.sqrt(4.0 ** 2 + 4.0 ** 2) / 5.0, rel=1e-15)
    # bf16-stored inputs: the float32 holder of a bf16 value is read exactly
    assert rel_fro(np.float32(1.0078125), np.float64(1.0)) == pytest.approx(0.0078125, rel=1e-15)
    # a zero reference returns the plain norm of the difference
    assert rel_fro(np.array([0.0, 2.0]), np.zeros(2)) == pytest.approx(2.0)


# ---------------------------------------------------------------- P3 GDN reduction

def test_scalar_gate_is_gated_deltanet():
    q, k, v, la, beta, S0 = rnd_inputs(5, T=16)
    la_head = la[..., 0]                                       # one gate per (b,t,h)
    la_b = np.repeat(la_head[..., None], la.shape[-1], axis=-1)
    o, S_T = oracle.kda_loop(q, k, v, la_b, beta, S0)
    o_g, S_g = oracle.gdn_loop(q, k, v, la_head, beta, S0)
    assert rel_fro(o, o_g) < 1e-12 and rel_fro(S_T, S_g) < 1e-12


# ---------------------------------------------------------------- P4 write-then-read

def test_write_then_read_returns_v():
    q, k, v, la, beta, S0 = rnd_inputs(6, T=10)
    o, _ = oracle.kda_loop(k, k, v, np.zeros_like(la), np.ones_like(beta), S0)
    assert np.abs(o - v).max() < 1e-12


# ---------------------------------------------------------------- P5 one-hot keys

def test_one_hot_keys_decouple_into_row_emas():
    rng = np.random.default_rng(7)
    B, T, H, dk, dv = 1, 30, 2, 4, 6
    idx = rng.integers(0, dk, (B, T, H))
    k = np.eye(dk)[idx]
    q = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    la = rng.uniform(-5, 0, (B, T, H, dk))
    beta = rng.uniform(0, 1, (B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, S_T = oracle.kda_loop(q, k, v, la, beta, S0)
    for h in range(H):
        S = S0[0, h].copy()
        for t in range(T):
            for c in range(dk):
                S[c] = math.exp(la[0, t, h, c]) * S[c]
            c = idx[0, t, h]
            S[c] = (1 - beta[0, t, h]) * S[c] + beta[0, t, h] * v[0, t, h]
            assert np.abs(o[0, t, h] - S.T @ q[0, t, h]).max() < 1e-12
        assert np.abs(S_T[0, h] - S).max() < 1e-12


# ---------------------------------------------------------------- P6 orthonormal keys

def test_orthonormal_keys_no_erasure():
    rng = np.random.default_rng(8)
    dk, dv, T = 8, 5, 8
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm.T[None, :, None, :]                                  # rows are orthonormal
    q = rng.standard_normal((1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    beta = rng.uniform(0, 1, (1, T, 1))
    o, _ = oracle.kda_loop(q, k, v, np.zeros((1, T, 1, dk)), beta, None)
    for t in range(T):
        ref = sum(beta[0, s, 0] * (q[0, t, 0] @ k[0, s, 0]) * v[0, s, 0] for s in range(t + 1))
        assert np.abs(o[0, t, 0] - ref).max() < 1e-12


# ---------------------------------------------------------------- P8 chunked form

@pytest.mark.parametrize("chunk", [1, 2, 4, 8, 16, 32, 64, 128])
@pytest.mark.parametrize("pairwise", [False, True])
def test_chunked_matches_loop(chunk, pairwise):
    if pairwise and chunk > 32:
        pytest.skip("pairwise form is O(C^2 dk) memory; checked on small chunks")
    x = rnd_inputs(9, B=1, T=150, H=2, dk=6, dv=4)
    o1, S1 = oracle.kda_loop(*x)
    o2, S2 = oracle.kda_chunked(*x, chunk=chunk, pairwise=pairwise)
    assert rel_fro(o2, o1) < 1e-11 and rel_fro(S2, S1) < 1e-11


def test_chunked_at_the_floor():
    """Every token at the floor: a 16-token tile reaches exactly -80 and a 64-chunk -320."""
    q, k, v, la, beta, S0 = rnd_inputs(10, B=1, T=96, H=2, dk=6, dv=4)
    la = np.full_like(la, -5.0)
    o1, S1 = oracle.kda_loop(q, k, v, la, beta, S0)
    for C in (16, 64):
        o2, S2 = oracle.kda_chunked(q, k, v, la, beta, S0, chunk=C)
        assert np.isfinite(o2).all() and rel_fro(o2, o1) < 1e-10 and rel_fro(S2, S1) < 1e-10


# ---------------------------------------------------------------- P9 split / resume

def test_split_resume():
    q, k, v, la, beta, S0 = rnd_inputs(11, T=40)
    o, S_T = oracle.kda_loop(q, k, v, la, beta, S0)
    o1, S_mid = oracle.kda_loop(q[:, :17], k[:, :17], v[:, :17], la[:, :17], beta[:, :17], S0)
    o2, S_end = oracle.kda_loop(q[:, 17:], k[:, 17:], v[:, 17:], la[:, 17:], beta[:, 17:], S_mid)
    assert rel_fro(np.concatenate([o1, o2], 1), o) < 1e-12 and rel_fro(S_end, S_T) < 1e-12


def test_decode_steps_equal_loop():
    q, k, v, la, beta, S0 = rnd_inputs(12, T=9)
    o, S_T = oracle.kda_loop(q, k, v, la, beta, S0)
    S = S0.copy()
    for t in range(q.shape[1]):
        ot, S = oracle.kda_decode_step(S, q[:, t], k[:, t], v[:, t], la[:, t], beta[:, t])
        assert np.abs(ot - o[:, t]).max() < 1e-12
    assert rel_fro(S, S_T) < 1e-12


# ---------------------------------------------------------------- P10 segments

def test_segment_composition_equals_full_run():
    q, k, v, la, beta, S0 = rnd_inputs(13, B=1, T=50, H=2)
    o, S_T = oracle.kda_loop(q, k, v, la, beta, S0)
    for seg in (7, 16, 50):
        o2, S2 = oracle.kda_segmented(q, k, v, la, beta, S0, seg_len=seg)
        assert rel_fro(o2, o) < 1e-11 and rel_fro(S2, S_T) < 1e-11


def test_segment_pairs_compose_associatively_and_naive_sum_fails():
    q, k, v, la, beta, S0 = rnd_inputs(14, B=1, T=48, H=1)
    pairs = oracle.segment_pairs(k[0, :, 0], v[0, :, 0], la[0, :, 0], beta[0, :, 0], 12)
    _, S_T = oracle.kda_loop(q, k, v, la, beta, None)
    left = oracle.compose(oracle.compose(pairs[3], pairs[2]), oracle.compose(pairs[1], pairs[0]))
    right = oracle.compose(pairs[3], oracle.compose(pairs[2], oracle.compose(pairs[1], pairs[0])))
    assert rel_fro(left[1], S_T[0, 0]) < 1e-12 and rel_fro(right[0], left[0]) < 1e-12
    naive = sum(p[1] for p in pairs)       # what plain linear attention could do; wrong for KDA
    assert rel_fro(naive, S_T[0, 0]) > 1e-2


def test_segment_transition_is_the_recurrence_on_identity():
    """By linearity in S0, running with S0 = I and v = 0 yields the transition matrix."""
    q, k, v, la, beta, _ = rnd_inputs(15, B=1, T=20, H=1, dk=5, dv=5)
    M = oracle.segment_transition(k[0, :, 0], la[0, :, 0], beta[0, :, 0])
    _, S = oracle.kda_loop(q, k, np.zeros_like(v), la, beta, np.eye(5)[None, None])
    assert rel_fro(M, S[0, 0]) < 1e-12


# ---------------------------------------------------------------- P11 structure

def test_linearity_in_v_and_state():
    q, k, v1, la, beta, S01 = rnd_inputs(16)
    _, _, v2, _, _, S02 = rnd_inputs(17)
    a, b = 0.7, -1.3
    o, S = oracle.kda_loop(q, k, a * v1 + b * v2, la, beta, a * S01 + b * S02)
    o1, Sa = oracle.kda_loop(q, k, v1, la, beta, S01)
    o2, Sb = oracle.kda_loop(q, k, v2, la, beta, S02)
    assert rel_fro(o, a * o1 + b * o2) < 1e-12 and rel_fro(S, a * Sa + b * Sb) < 1e-12


def test_value_columns_are_separable():
    q, k, v, la, beta, S0 = rnd_inputs(18, dv=6)
    o, S = oracle.kda_loop(q, k, v, la, beta, S0)
    cols = [1, 4]
    o2, S2 = oracle.kda_loop(q, k, v[..., cols], la, beta, S0[..., cols])
    assert rel_fro(o2, o[..., cols]) < 1e-12 and rel_fro(S2, S[..., cols]) < 1e-12


def test_head_and_batch_permutation_equivariance():
    q, k, v, la, beta, S0 = rnd_inputs(19, B=3, H=4)
    o, S = oracle.kda_loop(q, k, v, la, beta, S0)
    ph, pb = [2, 0, 3, 1], [1, 2, 0]
    xp = [x[pb][:, :, ph] for x in (q, k, v, la)]
    o2, S2 = oracle.kda_loop(*xp, beta[pb][:, :, ph], S0[pb][:, ph])
    assert rel_fro(o2, o[pb][:, :, ph]) < 1e-13 and rel_fro(S2, S[pb][:, ph]) < 1e-13


# ---------------------------------------------------------------- P12 non-expansiveness

def test_state_growth_bound():
    q, k, v, la, beta, S0 = rnd_inputs(20, B=1, H=1, T=60)
    S = S0
    for t in range(60):
        _, S_new = oracle.kda_decode_step(S, q[:, t], k[:, t], v[:, t], la[:, t], beta[:, t])
        bound = np.linalg.norm(S[0, 0], 2) + beta[0, t, 0] * np.linalg.norm(v[0, t, 0])
        assert np.linalg.norm(S_new[0, 0], 2) <= bound * (1 + 1e-12)
        S = S_new


# ---------------------------------------------------------------- P13 floor clamp

def test_floor_clamps_out_of_range_gates():
    q, k, v, la, beta, S0 = rnd_inputs(21, T=20)
    la_out = la.copy()
    la_out[:, ::3] = -9.0          # below the floor
    la_out[:, 1::5] = 0.4          # above 0 (no growth)
    la_in = np.minimum(np.maximum(la_out, -5.0), 0.0)
    o1, S1 = oracle.kda_loop(q, k, v, la_out, beta, S0)
    o2, S2 = oracle.kda_loop(q, k, v, la_in, beta, S0)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    # a wrong clamp would change the result: -9 is not -5
    o3, _ = oracle.kda_loop(q, k, v, np.where(la_out < -5, -9.0, la_in), beta, S0)
    assert np.array_equal(o3, o1)          # the oracle itself clamps -9 to -5
    assert oracle.floor_log_alpha(np.array([-9.0, -5.0, -1.0, 0.0, 0.4])).tolist() == [-5, -5, -1, 0, 0]


# ---------------------------------------------------------------- gate activation with a floor

def test_gate_from_logits_against_library_sigmoid():
    """-5 sigmoid(x): pinned to scipy's logistic function, its fixed point and both limits."""
    from scipy.special import expit
    x = np.linspace(-40.0, 40.0, 801)
    g = oracle.gate_from_logits(x)
    assert np.abs(g - (-5.0 * expit(x))).max() < 1e-14
    assert oracle.gate_from_logits(0.0) == -2.5                       # sigmoid(0) = 1/2 exactly
    assert oracle.gate_from_logits(800.0) == -5.0                     # the floor, reached in the limit
    assert oracle.gate_from_logits(-800.0) == 0.0                     # no decay in the other limit
    x = np.linspace(-30.0, 30.0, 601)                                  # sigmoid(x) < 1 in float64
    g = oracle.gate_from_logits(x)
    assert np.all(np.diff(g) < 0) and np.all((g > -5.0) & (g < 0.0))
    # inside [-5, 0] already: the clamp of the recurrence changes nothing
    assert np.array_equal(oracle.floor_log_alpha(g), g)


# ---------------------------------------------------------------- speculative verify / commit

def test_decode_verify_matches_bruteforce_and_keeps_state():
    q, k, v, la, beta, S0 = rnd_inputs(21, B=3, T=6, H=2)
    S_keep = S0.copy()
    o = oracle.kda_decode_verify(S0, q, k, v, la, beta)
    o_bf, _ = oracle.kda_bruteforce(q, k, v, la, beta, S0)
    assert rel_fro(o, o_bf) < 1e-12
    assert np.array_equal(S0, S_keep)


def test_decode_commit_matches_bruteforce_prefixes():
    q, k, v, la, beta, S0 = rnd_inputs(22, B=5, T=6, H=2)
    n_accept = [0, 3, 6, 9, -2]                                        # 9 and -2 are clamped
    S = oracle.kda_decode_commit(S0, q, k, v, la, beta, n_accept)
    for i, m in enumerate(n_accept):
        m = min(max(m, 0), 6)
        if m == 0:
            assert np.array_equal(S[i], S0[i])
            continue
        sl = slice(i, i + 1)
        _, S_bf = oracle.kda_bruteforce(q[sl, :m], k[sl, :m], v[sl, :m], la[sl, :m], beta[sl, :m], S0[sl])
        assert rel_fro(S[i], S_bf[0]) < 1e-12


# ---------------------------------------------------------------- optional q/k L2 normalisation

def test_l2_normalize_against_library_and_closed_form():
    from sklearn.preprocessing import normalize
    rng = np.random.default_rng(31)
    x = rng.standard_normal((7, 5, 33)) * rng.uniform(0.01, 30.0, (7, 5, 1))
    flat = x.reshape(-1, 33)
    assert np.abs(oracle.l2_normalize(flat, eps=0.0) - normalize(flat)).max() < 1e-15
    y = oracle.l2_normalize(x)
    s = np.sum(x * x, axis=-1)
    assert np.abs(np.linalg.norm(y, axis=-1) - np.sqrt(s / (s + oracle.QK_NORM_EPS))).max() < 1e-14
    assert np.array_equal(oracle.l2_normalize(np.zeros((2, 16))), np.zeros((2, 16)))   # finite at zero


def test_normalised_keys_write_then_read_any_length():
    """alpha = beta = 1 and q = k: with k normalised inside, o_t = v_t for keys of any length
    (the erase / write algebra needs unit keys, which the normalisation supplies)."""
    q, k, v, la, beta, S0 = rnd_inputs(32, T=10, unit_k=False)
    k = k * np.random.default_rng(33).uniform(0.2, 9.0, k.shape[:-1] + (1,))
    kn = oracle.l2_normalize(k, eps=0.0)
    o, _ = oracle.kda_loop(kn, kn, v, np.zeros_like(la), np.ones_like(beta), S0)
    assert np.abs(o - v).max() < 1e-12
