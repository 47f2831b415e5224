"""CPU oracle for the Kimi Delta Attention (KDA) hot path -- TEST INFRASTRUCTURE.

Only tests/, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this module.  The library's product path never calls it, and
it shares no code with the HIP kernels or their bindings.

Everything here is plain numpy in float64.  Inputs are read as stored (bf16
values arrive as float32 arrays holding exactly the bf16 numbers) and upcast
exactly, so the oracle sees the same numbers as the GPU.

Sources (web pages; section names translated from Korean):

* [P1] orkas.ai, "Kimi K3 architecture" deep-read, section "Sequence: three
  quarters of the layers stopped reading everything" -- a fixed-size recurrent
  state kept like a memo instead of re-reading the prefix; decay makes recent
  tokens weigh more.
* [P1-floor] same page, section "The floor that removed a GPU code path" --
  chunked evaluation divides by a cumulative decay (a product of numbers
  below one); the log-decay is floored so that each step keeps at least
  0.67 % (natural log -5), a 16-token tile's cumulative log-decay stays in
  (-80, 0), its reciprocal stays below e^80 ~ 5.5e34, inside bf16's range.
* [P1-serve] same page, section "The cost comes back in the serving stack" --
  the state is updated sequentially and in place; zero-start states cannot be
  summed; each segment splits into (cumulative transition, zero-start state),
  which compose, and a prefix scan recovers every segment's start state.
* [P1-act] same page, section "The floor that removed a GPU code path", read
  backwards: the hardware's range fixed the tile interval, the interval fixed
  the constant, and the constant made the gate's activation function need a
  floor.
* [P1-spec] same page, section "The cost comes back in the serving stack",
  speculative decoding: the state is updated in place, so a rejected draft
  cannot be rolled back; the per-token projection inputs, far smaller than the
  state, are cached instead and the state is rebuilt from them on chip.
* [P4-1] llm-wiki.hwlabs.dev, "Kimi K3 ... linear attention", section
  "1. Limits of softmax attention and KDA's direction" -- a fixed-size state
  matrix S is updated with each new token and the query is multiplied by S.
* [P4-GDN] same page, section "Difference between GatedDeltaNet and KDA" --
  GatedDeltaNet gates decay with one scalar per head; KDA gives every
  feature (channel) dimension its own gate.
* [P3-key] allinfo.ai.kr, "Kimi K3 structure analysis", section "Key
  messages" -- KDA is Gated DeltaNet plus a per-channel decay layer.

None of the pages prints the recurrence; the page in [P4] lists the exact KDA
formula as still unpublished ("Open question").  The oracle implements the
gated delta rule with per-channel decay in its plainest form:

    g_t   = min(max(log_alpha_t, -5), 0)              (per key channel)
    S_t   = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
    o_t   = S_t^T q_t

S is [dk, dv]: rows are key channels (the decay axis), columns value channels.
Readings taken where the pages are silent: decay before the delta update; the
output reads the post-update state; no 1/sqrt(dk) scale, no output gate; the
upper clamp at 0 (the pages call decay factors numbers below one).

Parity pins: every function here is checked in tests/test_oracle_pins.py
against closed forms, independently written reductions, exact rational
arithmetic and invariants.  Equality with Moonshot's own (unpublished) KDA is
parity unpinned.
"""
from __future__ import annotations

import numpy as np

LOG_ALPHA_FLOOR = -5.0   # [P1-floor]: each step keeps >= e^-5 ~ 0.67 %
SUBTILE = 16             # [P1-floor]: the tile length whose range the floor bounds


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def floor_log_alpha(log_alpha):
    """Clamp the log-decay to [-5, 0] ([P1-floor]; the upper bound 0 is our reading)."""
    return np.minimum(np.maximum(_f64(log_alpha), LOG_ALPHA_FLOOR), 0.0)


def gate_from_logits(x):
    """Log-decay from raw gate logits through an activation floored at -5 ([P1-act]).

    The pages name no formula.  Reading: the plainest bounded activation with that floor,
    g = -5 * sigmoid(x) = -5 / (1 + e^-x), which lies in (-5, 0) (the clamp of
    floor_log_alpha then changes nothing).  Large logits decay fastest.
    """
    x = _f64(x)
    with np.errstate(over="ignore"):
        return LOG_ALPHA_FLOOR / (1.0 + np.exp(-x))


QK_NORM_EPS = 1e-6


def l2_normalize(x, eps=QK_NORM_EPS):
    """Optional per-token normalisation of q and k over the dk channels: x / sqrt(sum x^2 + eps).

    The pages leave normalisation to the model (no formula is printed); this is the common
    form, with a small epsilon so that a zero vector stays finite.  Applied, when asked for,
    to q and k as stored, before every other step.
    """
    x = _f64(x)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def _bhtd(x):
    """[B,T,H,D] -> [B,H,T,D] view."""
    return np.swapaxes(x, 1, 2)


def kda_loop(q, k, v, log_alpha, beta, S0=None):
    """Token-by-token recurrence ([P4-1], [P4-GDN]).

    q, k, log_alpha: [B,T,H,dk]; v: [B,T,H,dv]; beta: [B,T,H]; S0: [B,H,dk,dv] or None.
    Returns o [B,T,H,dv] and S_T [B,H,dk,dv], both float64.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    alpha = np.exp(floor_log_alpha(log_alpha))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.empty((B, T, H, dv))
    for t in range(T):
        S *= alpha[:, t, :, :, None]                              # Diag(alpha_t) S
        kt = k[:, t]                                              # [B,H,dk]
        pred = np.einsum("bhcj,bhc->bhj", S, kt)                  # S^T k_t
        S += beta[:, t, :, None, None] * kt[..., None] * (v[:, t] - pred)[:, :, None, :]
        o[:, t] = np.einsum("bhcj,bhc->bhj", S, q[:, t])          # S_t^T q_t
    return o, S


def kda_decode_step(state, q, k, v, log_alpha, beta):
    """One recurrent step for N independent sequences ([P4-1]: O(1) state).

    state [N,H,dk,dv]; q, k, log_alpha [N,H,dk]; v [N,H,dv]; beta [N,H].
    Returns (o [N,H,dv], new_state), float64; the input is not modified.
    """
    o, S = kda_loop(_f64(q)[:, None], _f64(k)[:, None], _f64(v)[:, None],
                    _f64(log_alpha)[:, None], _f64(beta)[:, None], state)
    return o[:, 0], S


def kda_decode_verify(state, q, k, v, log_alpha, beta):
    """Speculative-decoding verify ([P1-spec]): the outputs of n draft tokens per sequence,
    draft j read from the state advanced through drafts 0..j, with the caller's state left as
    it was (an in-place update could not be rolled back after a rejection).

    state [N,H,dk,dv]; q, k, log_alpha [N,n,H,dk]; v [N,n,H,dv]; beta [N,n,H].
    Returns o [N,n,H,dv] float64.
    """
    o, _ = kda_loop(q, k, v, log_alpha, beta, state)
    return o


def kda_decode_commit(state, q, k, v, log_alpha, beta, n_accept):
    """Commit after verification ([P1-spec]): the state of sequence i advanced by its first
    n_accept[i] draft tokens (clamped to [0, n]), replayed from the cached per-token inputs.

    Shapes as kda_decode_verify; n_accept [N] integers.  Returns the new state [N,H,dk,dv]
    float64; the input is not modified.
    """
    out = _f64(state).copy()
    n = np.shape(q)[1]
    for i, m in enumerate(np.asarray(n_accept).reshape(-1)):
        m = min(max(int(m), 0), n)
        if m:
            _, S = kda_loop(_f64(q)[i:i + 1, :m], _f64(k)[i:i + 1, :m], _f64(v)[i:i + 1, :m],
                            _f64(log_alpha)[i:i + 1, :m], _f64(beta)[i:i + 1, :m], out[i:i + 1])
            out[i] = S[0]
    return out


def kda_bruteforce(q, k, v, log_alpha, beta, S0=None):
    """Explicit matrix products, for T <= 8: an independent check of kda_loop.

    P_t = (I - beta_t k_t k_t^T) Diag(alpha_t);  S_t = P_t...P_1 S0 + sum_s P_t...P_{s+1} beta_s k_s v_s^T.
    """
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    alpha = np.exp(floor_log_alpha(log_alpha))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert T <= 8, "brute force is for tiny T"
    S0 = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0)
    o = np.empty((B, T, H, dv))
    S_T = np.empty((B, H, dk, dv))
    eye = np.eye(dk)
    for b in range(B):
        for h in range(H):
            P = [(eye - beta[b, t, h] * np.outer(k[b, t, h], k[b, t, h])) @ np.diag(alpha[b, t, h])
                 for t in range(T)]
            for t in range(T):
                prod = eye
                for s in range(t, -1, -1):
                    prod = prod @ P[s]
                St = prod @ S0[b, h]
                for s in range(t + 1):
                    tail = eye
                    for r in range(t, s, -1):
                        tail = tail @ P[r]
                    St = St + tail @ (beta[b, s, h] * np.outer(k[b, s, h], v[b, s, h]))
                o[b, t, h] = St.T @ q[b, t, h]
                if t == T - 1:
                    S_T[b, h] = St
    return o, S_T


def kda_chunked(q, k, v, log_alpha, beta, S0=None, chunk=64, pairwise=False):
    """Chunkwise form: the same recurrence evaluated C tokens at a time.

    Within a chunk of C tokens with start state S, with Gamma_t the inclusive
    cumulative sum of the floored log-decay ([P1-floor]: chunked evaluation
    divides by the cumulative decay):

        Kt = k * e^Gamma,  Qt = q * e^Gamma,  Kh = k * e^(Gamma_C - Gamma)
        A[t,s] = sum_c k[t,c] k[s,c] e^(Gamma[t,c]-Gamma[s,c])   (s <  t)
        M[t,s] = sum_c q[t,c] k[s,c] e^(Gamma[t,c]-Gamma[s,c])   (s <= t)
        U      = (I + Diag(beta) A)^-1 Diag(beta) (V - Kt S)
        O      = Qt S + M U
        S'     = Diag(e^Gamma_C) S + Kh^T U

    No sub-tiling: float64 holds e^(5*C) for C <= 128.  With ``pairwise``
    the decay-weighted products A and M are summed per position pair instead
    of factorised as (k e^Gamma)(k e^-Gamma)^T -- the pages' description of the
    earlier generation's diagonal tiles ([P1-floor]).
    """
    q, k, v = _bhtd(_f64(q)), _bhtd(_f64(k)), _bhtd(_f64(v))
    beta = np.swapaxes(_f64(beta), 1, 2)                      # [B,H,T]
    g_all = _bhtd(floor_log_alpha(log_alpha))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if S0 is None else _f64(S0).copy()
    o = np.empty((B, H, T, dv))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        C = t1 - t0
        qc, kc, vc, bc = q[:, :, t0:t1], k[:, :, t0:t1], v[:, :, t0:t1], beta[:, :, t0:t1]
        G = np.cumsum(g_all[:, :, t0:t1], axis=2)                 # [B,H,C,dk]
        GC = G[:, :, -1]                                          # [B,H,dk]
        Kt = kc * np.exp(G)
        Qt = qc * np.exp(G)
        Kh = kc * np.exp(GC[:, :, None, :] - G)
        if pairwise:
            D = np.exp(G[:, :, :, None, :] - G[:, :, None, :, :])  # [B,H,t,s,dk]
            A = np.einsum("bhtc,bhsc,bhtsc->bhts", kc, kc, D)
            M = np.einsum("bhtc,bhsc,bhtsc->bhts", qc, kc, D)
        else:
            Kinv = kc * np.exp(-G)
            A = Kt @ np.swapaxes(Kinv, -1, -2)
            M = Qt @ np.swapaxes(Kinv, -1, -2)
        A = np.tril(A, -1)
        M = np.tril(M, 0)
        Lmat = np.eye(C) + bc[..., :, None] * A
        rhs = bc[..., :, None] * (vc - Kt @ S)
        U = np.linalg.solve(Lmat, rhs)
        o[:, :, t0:t1] = Qt @ S + M @ U
        S = np.exp(GC)[..., :, None] * S + np.swapaxes(Kh, -1, -2) @ U
    return np.swapaxes(o, 1, 2), S


def gla_loop(q, k, v, log_alpha, S0=None):
    """Gated linear attention with per-channel decay, written independently:
    S_t = Diag(alpha_t) S_{t-1} + k_t v_t^T,  o_t = S_t^T q_t."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    a = np.exp(floor_log_alpha(log_alpha))
    B, T, H, dk = q.shape
    out = np.empty(v.shape[:3] + (v.shape[-1],))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, v.shape[-1])) if S0 is None else _f64(S0)[b, h].copy()
            for t in range(T):
                S = a[b, t, h][:, None] * S + np.outer(k[b, t, h], v[b, t, h])
                out[b, t, h] = S.T @ q[b, t, h]
    return out


def gdn_loop(q, k, v, log_alpha_head, beta, S0=None):
    """Gated DeltaNet with one scalar gate per head ([P4-GDN]), written independently:
    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t.
    log_alpha_head: [B,T,H] (floored like KDA's)."""
    q, k, v, beta = _f64(q), _f64(k), _f64(v), _f64(beta)
    a = np.exp(floor_log_alpha(log_alpha_head))
    B, T, H, dk = q.shape
    out = np.empty(v.shape)
    S_out = np.empty((B, H, dk, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, v.shape[-1])) if S0 is None else _f64(S0)[b, h].copy()
            for t in range(T):
                kk = k[b, t, h]
                S = a[b, t, h] * ((np.eye(dk) - beta[b, t, h] * np.outer(kk, kk)) @ S) \
                    + beta[b, t, h] * np.outer(kk, v[b, t, h])
                out[b, t, h] = S.T @ q[b, t, h]
            S_out[b, h] = S
    return out, S_out


# ---------------------------------------------------------------------------
# Segment decomposition ([P1-serve]): each segment becomes a pair
# (cumulative transition M, zero-start state S_loc) with S_end = M S_start + S_loc.
# ---------------------------------------------------------------------------

def segment_transition(k, log_alpha, beta):
    """Cumulative transition of one segment for one (batch, head):
    M = P_T ... P_1 with P_t = (I - beta_t k_t k_t^T) Diag(alpha_t).
    k, log_alpha: [T, dk]; beta: [T].  Returns [dk, dk]."""
    k, beta = _f64(k), _f64(beta)
    a = np.exp(floor_log_alpha(log_alpha))
    dk = k.shape[1]
    M = np.eye(dk)
    for t in range(k.shape[0]):
        M = ((np.eye(dk) - beta[t] * np.outer(k[t], k[t])) * a[t][None, :]) @ M
    return M


def segment_pairs(k, v, log_alpha, beta, seg_len):
    """(M, S_loc) per segment for one (batch, head).  k, log_alpha [T,dk]; v [T,dv]; beta [T]."""
    T = k.shape[0]
    pairs = []
    for s0 in range(0, T, seg_len):
        s1 = min(T, s0 + seg_len)
        M = segment_transition(k[s0:s1], log_alpha[s0:s1], beta[s0:s1])
        _, S_loc = kda_loop(*(x[None, s0:s1, None] for x in (k, k, v, log_alpha)),
                            _f64(beta)[None, s0:s1, None], None)
        pairs.append((M, S_loc[0, 0]))
    return pairs


def compose(pair2, pair1):
    """(M2, S2) o (M1, S1) = (M2 M1, M2 S1 + S2): run segment 1, then segment 2."""
    M2, S2 = pair2
    M1, S1 = pair1
    return M2 @ M1, M2 @ S1 + S2


def segment_start_states(pairs, S0):
    """Prefix scan over segment pairs: the start state of every segment, and the end state."""
    starts = []
    S = _f64(S0)
    for M, S_loc in pairs:
        starts.append(S)
        S = M @ S + S_loc
    return starts, S


def kda_segmented(q, k, v, log_alpha, beta, S0=None, seg_len=256):
    """Two-pass evaluation via segment pairs, for one or more (batch, head):
    pass 1 builds (M, S_loc) per segment, a prefix scan gives start states,
    pass 2 reruns each segment from its true start state.  Same layouts as kda_loop."""
    q, k, v, log_alpha, beta = (_f64(x) for x in (q, k, v, log_alpha, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.empty((B, T, H, dv))
    S_T = np.empty((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            pairs = segment_pairs(k[b, :, h], v[b, :, h], log_alpha[b, :, h], beta[b, :, h], seg_len)
            s_init = np.zeros((dk, dv)) if S0 is None else _f64(S0)[b, h]
            starts, S_T[b, h] = segment_start_states(pairs, s_init)
            for i, s0 in enumerate(range(0, T, seg_len)):
                s1 = min(T, s0 + seg_len)
                oi, _ = kda_loop(*(x[None, s0:s1, None] for x in (q[b, :, h], k[b, :, h], v[b, :, h],
                                                                     log_alpha[b, :, h])),
                                 beta[b, s0:s1, h][None, :, None], starts[i][None, None])
                o[b, s0:s1, h] = oi[0, :, 0]
    return o, S_T


def rel_fro(x, ref):
    """Relative Frobenius error ||x - ref|| / ||ref|| over a whole tensor, in float64."""
    x, ref = _f64(x), _f64(ref)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((x - ref).ravel())
    return num / den if den > 0 else num
