"""Seeded synthetic inputs for the KDA hot path.

This module is the only code shared by the CPU oracle and the GPU path's tests
and benchmark.  It draws random tensors and nothing else: it holds none of the
recurrence's arithmetic (no decay, no cumulative sums, no delta rule).

Generator: numpy's Philox (4x64, 10 rounds) keyed per block, so any
(batch, head, token-block) slice of any tensor can be regenerated on its own:

    key = (tag << 8 | tensor_id,  b << 40 | h << 20 | block)

with ``tag = 0x4B4441 * 16 + workload id`` and blocks of 65,536 tokens.

Input recipes (one per workload; the shapes are the five workloads this
library is measured on, see ``WORKLOADS``):

* q, k: N(0,1), L2-normalised over the key dimension in float32 (no epsilon),
  then rounded to the storage dtype.
* v: N(0,1).
* beta: sigmoid(N(0, s^2)).
* log_alpha: either -5 * sigmoid(N(0, 1.5^2)), or Uniform[-5, 0) with a
  fraction of tokens pinned at exactly -5 on every head and channel (a
  Bernoulli draw per (batch, token)).
* S0 / decode state: N(0, s^2) float32, or zeros.

bfloat16 storage is represented here as float32 arrays holding exactly
bf16-representable values (round to nearest even), so the oracle and the GPU
see identical numbers.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

BLOCK_T = 65536
TAG_BASE = 0x4B4441 * 16

# tensor ids used in the Philox key
T_Q, T_K, T_V, T_LOGA, T_BETA, T_STATE, T_PIN = 0, 1, 2, 3, 4, 5, 6


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return (rounded.astype(np.uint32)).view(np.float32).reshape(x.shape)


def _gen(tag: int, tensor_id: int, b: int, h: int, blk: int) -> np.random.Generator:
    assert 0 <= b < (1 << 24) and 0 <= h < (1 << 20) and 0 <= blk < (1 << 20)
    key = [((tag << 8) | tensor_id) & 0xFFFFFFFFFFFFFFFF, (b << 40) | (h << 20) | blk]
    return np.random.Generator(np.random.Philox(key=key))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


@dataclass(frozen=True)
class Recipe:
    """Shape and value distributions of one prefill/decode workload."""
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    chunk: int
    dtype: str                      # "f32" or "bf16": storage of q, k, v, o
    qk: str = "l2"                  # "l2": q, k ~ N(0,1) L2-normalised per token; "raw": not normalised
    loga: str = "sig15"             # "sig15": -5*sigmoid(N(0,1.5^2)); "unif": U[-5,0);
                                    # "logit15": raw gate logits N(0,1.5^2) (the log-decay is
                                    # formed from them by the code under test)
    pin_frac: float = 0.0           # fraction of tokens with log_alpha pinned at -5
    beta_std: float = 1.0           # beta = sigmoid(N(0, beta_std^2))
    s0_std: float = 0.0             # 0 => S0 is None (zeros)
    tag: int = TAG_BASE
    steps: int = 0                  # decode workloads: number of consecutive steps

    def with_shape(self, **kw) -> "Recipe":
        return replace(self, **kw)


WORKLOADS = {
    0: Recipe("kda_fwd_tiny_f32", B=1, T=64, H=2, dk=16, dv=16, chunk=16, dtype="f32",
              tag=TAG_BASE + 0),
    1: Recipe("kda_prefill_b1_t4096_h16", B=1, T=4096, H=16, dk=128, dv=128, chunk=64,
              dtype="bf16", s0_std=0.01, tag=TAG_BASE + 1),
    2: Recipe("kda_prefill_b8_t8192_h32_floor_stress", B=8, T=8192, H=32, dk=128, dv=128,
              chunk=64, dtype="bf16", loga="unif", pin_frac=0.25, beta_std=2.0,
              tag=TAG_BASE + 2),
    3: Recipe("kda_prefill_b1_t1m_h32", B=1, T=1 << 20, H=32, dk=128, dv=128, chunk=64,
              dtype="bf16", tag=TAG_BASE + 3),
    4: Recipe("kda_decode_n256_h32", B=256, T=64, H=32, dk=128, dv=128, chunk=64,
              dtype="bf16", loga="unif", s0_std=0.05, tag=TAG_BASE + 4, steps=64),
}


def _blocks(T: int):
    for blk in range((T + BLOCK_T - 1) // BLOCK_T):
        t0 = blk * BLOCK_T
        yield blk, t0, min(T, t0 + BLOCK_T)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(x) if dtype == "bf16" else x.astype(np.float32)


def gen_head(r: Recipe, name: str, b: int, h: int, t0: int = 0, t1: int | None = None) -> np.ndarray:
    """Values of tensor ``name`` for one (batch, head) over tokens [t0, t1).

    Returns [t1-t0, D] float32 ([t1-t0] for beta).  Blocks are generated whole
    and sliced, so any sub-range is consistent with the full tensor.
    """
    t1 = r.T if t1 is None else t1
    out = []
    for blk, b0, b1 in _blocks(r.T):
        if b1 <= t0 or b0 >= t1:
            continue
        full = _gen_block(r, name, b, h, blk, b1 - b0)
        out.append(full[max(t0, b0) - b0: min(t1, b1) - b0])
    return np.concatenate(out, axis=0)


def _pin_mask(r: Recipe, b: int, blk: int, n: int) -> np.ndarray:
    g = _gen(r.tag, T_PIN, b, 0, blk)
    return g.random(n, dtype=np.float32) < np.float32(r.pin_frac)


def _gen_block(r: Recipe, name: str, b: int, h: int, blk: int, n: int) -> np.ndarray:
    if name in ("q", "k"):
        g = _gen(r.tag, T_Q if name == "q" else T_K, b, h, blk)
        x = g.standard_normal((n, r.dk), dtype=np.float32)
        if r.qk == "raw":                    # unnormalised (for the in-kernel normalisation)
            return _store(x, r.dtype)
        nrm = np.sqrt(np.sum(x * x, axis=1, dtype=np.float32), dtype=np.float32)
        return _store(x / nrm[:, None], r.dtype)
    if name == "v":
        g = _gen(r.tag, T_V, b, h, blk)
        return _store(g.standard_normal((n, r.dv), dtype=np.float32), r.dtype)
    if name == "beta":
        g = _gen(r.tag, T_BETA, b, h, blk)
        return _sigmoid(np.float32(r.beta_std) * g.standard_normal(n, dtype=np.float32))
    if name == "log_alpha":
        g = _gen(r.tag, T_LOGA, b, h, blk)
        if r.loga == "sig15":
            x = np.float32(-5.0) * _sigmoid(np.float32(1.5) * g.standard_normal((n, r.dk), dtype=np.float32))
        elif r.loga == "unif":
            x = np.float32(-5.0) + np.float32(5.0) * g.random((n, r.dk), dtype=np.float32)
        elif r.loga == "logit15":
            if r.pin_frac > 0:
                raise ValueError("pinned log-decays are not defined for raw logits")
            x = np.float32(1.5) * g.standard_normal((n, r.dk), dtype=np.float32)
        else:
            raise ValueError(r.loga)
        if r.pin_frac > 0:
            x[_pin_mask(r, b, blk, n)] = np.float32(-5.0)
        return x.astype(np.float32)
    raise KeyError(name)


def gen_state(r: Recipe, b: int, h: int) -> np.ndarray:
    """S0 (prefill) or the initial decode state for one (batch, head): [dk, dv] float32."""
    g = _gen(r.tag, T_STATE, b, h, 0)
    return (np.float32(r.s0_std) * g.standard_normal((r.dk, r.dv), dtype=np.float32)).astype(np.float32)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_prefill(r: Recipe, heads: list[int] | None = None) -> dict:
    """Full prefill inputs as float32 numpy arrays in the library's layouts.

    q, k, log_alpha: [B,T,H,dk]; v: [B,T,H,dv]; beta: [B,T,H]; S0: [B,H,dk,dv] or None.
    ``heads`` restricts generation to a subset of heads (others left zero).
    """
    B, T, H = r.B, r.T, r.H
    heads = list(range(H)) if heads is None else heads
    out = {
        "q": np.zeros((B, T, H, r.dk), np.float32),
        "k": np.zeros((B, T, H, r.dk), np.float32),
        "v": np.zeros((B, T, H, r.dv), np.float32),
        "log_alpha": np.zeros((B, T, H, r.dk), np.float32),
        "beta": np.zeros((B, T, H), np.float32),
    }
    jobs = [(name, b, h) for name in out for b in range(B) for h in heads]

    def run(job):
        name, b, h = job
        out[name][b, :, h] = gen_head(r, name, b, h)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(run, jobs))
    if r.s0_std > 0:
        S0 = np.zeros((B, H, r.dk, r.dv), np.float32)
        for b in range(B):
            for h in heads:
                S0[b, h] = gen_state(r, b, h)
        out["S0"] = S0
    else:
        out["S0"] = None
    return out


def make_decode(r: Recipe) -> dict:
    """Decode inputs: state [N,H,dk,dv] and per-step tensors with a leading step axis.

    Step s of the decode sequence uses token s of the prefill-layout tensors,
    so q[s] == prefill q[:, s] and 'steps' decode calls equal one prefill of
    T = steps from the same state.
    """
    rr = r.with_shape(T=r.steps)
    pre = make_prefill(rr.with_shape(s0_std=0.0))
    state = np.zeros((r.B, r.H, r.dk, r.dv), np.float32)
    for n in range(r.B):
        for h in range(r.H):
            state[n, h] = gen_state(r, n, h)
    return {
        "state": state,
        "q": np.ascontiguousarray(pre["q"].transpose(1, 0, 2, 3)),
        "k": np.ascontiguousarray(pre["k"].transpose(1, 0, 2, 3)),
        "v": np.ascontiguousarray(pre["v"].transpose(1, 0, 2, 3)),
        "log_alpha": np.ascontiguousarray(pre["log_alpha"].transpose(1, 0, 2, 3)),
        "beta": np.ascontiguousarray(pre["beta"].transpose(1, 0, 2)),
    }


def make_prefill_device(r: Recipe, device, keyed_heads=()) -> dict:
    """Prefill inputs generated straight into device tensors, for workloads whose float32 host
    copies would not fit (T = 1M x 32 heads is 17 GB per tensor).

    Heads in ``keyed_heads`` hold exactly the keyed values of ``gen_head`` (the oracle can
    regenerate them); every other head is drawn on the device by torch's generator, seeded
    from the workload's tag, with the same recipe.  Returns torch tensors in the library's
    layouts and storage dtypes: q, k, v ([B,T,H,d], bf16 or f32), log_alpha, beta (f32),
    S0 (f32 or None).
    """
    import torch
    if r.pin_frac > 0:
        raise ValueError("pinned-floor recipes are generated on the host (make_prefill)")
    dt = torch.bfloat16 if r.dtype == "bf16" else torch.float32
    B, T, H = r.B, r.T, r.H
    out = {
        "q": torch.empty((B, T, H, r.dk), dtype=dt, device=device),
        "k": torch.empty((B, T, H, r.dk), dtype=dt, device=device),
        "v": torch.empty((B, T, H, r.dv), dtype=dt, device=device),
        "log_alpha": torch.empty((B, T, H, r.dk), dtype=torch.float32, device=device),
        "beta": torch.empty((B, T, H), dtype=torch.float32, device=device),
    }
    store = {"q": dt, "k": dt, "v": dt, "log_alpha": torch.float32, "beta": torch.float32}
    keyed = set(keyed_heads)
    gen = torch.Generator(device=device)
    gen.manual_seed(r.tag)
    for b in range(B):
        for h in range(H):
            for name in out:
                if h in keyed:
                    out[name][b, :, h] = torch.from_numpy(gen_head(r, name, b, h)).to(device, store[name])
                    continue
                for t0, t1 in ((0, T),):              # one draw per head: few launches
                    n = t1 - t0
                    if name in ("q", "k"):
                        x = torch.randn((n, r.dk), generator=gen, device=device, dtype=torch.float32)
                        if r.qk != "raw":
                            x = x / torch.sqrt((x * x).sum(dim=1, keepdim=True))
                    elif name == "v":
                        x = torch.randn((n, r.dv), generator=gen, device=device, dtype=torch.float32)
                    elif name == "beta":
                        x = torch.sigmoid(r.beta_std * torch.randn(n, generator=gen, device=device,
                                                                   dtype=torch.float32))
                    elif r.loga == "sig15":
                        x = -5.0 * torch.sigmoid(1.5 * torch.randn((n, r.dk), generator=gen, device=device,
                                                                   dtype=torch.float32))
                    elif r.loga == "logit15":
                        x = 1.5 * torch.randn((n, r.dk), generator=gen, device=device, dtype=torch.float32)
                    else:
                        x = -5.0 + 5.0 * torch.rand((n, r.dk), generator=gen, device=device, dtype=torch.float32)
                    out[name][b, t0:t1, h] = x.to(store[name])
    if r.s0_std > 0:
        S0 = torch.empty((B, H, r.dk, r.dv), dtype=torch.float32, device=device)
        for b in range(B):
            for h in range(H):
                S0[b, h] = torch.from_numpy(gen_state(r, b, h)).to(device)
        out["S0"] = S0
    else:
        out["S0"] = None
    return out
