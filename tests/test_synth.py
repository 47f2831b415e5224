"""The seeded input generator: determinism, slice consistency, recipes."""
import numpy as np
import pytest

import kda_synth as ks


def test_round_bf16_matches_torch():
    import torch
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10.0
    x[:4] = [0.0, -0.0, 1e-40, 3.0e38]
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ks.round_bf16(x), ref)


def test_keyed_regeneration_and_slices():
    r = ks.WORKLOADS[1].with_shape(T=70000, H=2)     # two token blocks
    full = ks.gen_head(r, "k", 0, 1)
    part = ks.gen_head(r, "k", 0, 1, 65000, 66000)   # straddles the block boundary
    assert np.array_equal(part, full[65000:66000])
    assert np.array_equal(ks.gen_head(r, "k", 0, 1), full)
    assert not np.array_equal(ks.gen_head(r, "k", 0, 0)[:10], full[:10])
    assert not np.array_equal(ks.gen_head(r, "q", 0, 1)[:10], full[:10])


def test_recipes():
    r = ks.WORKLOADS[2].with_shape(B=2, T=4096, H=2)
    x = ks.make_prefill(r)
    la = x["log_alpha"]
    assert la.min() >= -5.0 and la.max() < 0.0
    pinned = np.all(la == -5.0, axis=(2, 3))                   # per (b, t)
    assert 0.22 < pinned.mean() < 0.28
    nrm = np.linalg.norm(x["k"].astype(np.float64), axis=-1)
    assert np.abs(nrm - 1).max() < 2 ** -6
    assert x["S0"] is None
    assert np.array_equal(ks.round_bf16(x["q"]), x["q"])       # bf16-representable
    r0 = ks.WORKLOADS[0]
    x0 = ks.make_prefill(r0)
    assert x0["q"].shape == (1, 64, 2, 16) and x0["beta"].shape == (1, 64, 2)
    assert (x0["log_alpha"] <= 0).all() and (x0["log_alpha"] >= -5).all()


def test_decode_steps_are_prefill_tokens():
    r = ks.WORKLOADS[4].with_shape(B=3, H=2, steps=5)
    d = ks.make_decode(r)
    p = ks.make_prefill(r.with_shape(T=5, s0_std=0.0))
    assert np.array_equal(d["q"][2], p["q"][:, 2])
    assert d["state"].shape == (3, 2, 128, 128)
    assert 0.045 < d["state"].std() < 0.055
