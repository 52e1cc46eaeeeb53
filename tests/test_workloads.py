"""The seeded input generator: determinism, rounding, planted structure (CPU)."""

import hashlib

import numpy as np
import torch

from workloads import WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, make_base, make_step
from workloads.configs import scaled


def _h(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_bf16_rounding_matches_torch_rne():
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 100
    x[:4] = [1.00390625, 1.01171875, -3.0078125, 0.0]  # exact ties in bf16
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(x), ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_step_dependent():
    w = scaled(WORKLOADS["llada8b_8k"], seq_len=512, q_heads=4, kv_heads=4)
    a, b = make_step(w, 3), make_step(w, 3)
    for n in "qkv":
        assert _h(a[n]) == _h(b[n])
        assert a[n].dtype == np.uint16 and a[n].shape == (1, 4, 512, 128)
    c = make_step(w, 4)
    assert _h(a["q"]) != _h(c["q"]) and _h(a["k"]) != _h(c["k"])
    assert _h(a["v"]) == _h(c["v"])  # the walk leaves V fixed


def test_fresh_qv_noise_keeps_k():
    w = WORKLOADS["tiny_fp32_h4_l512"]
    base = make_base(w)
    s1, s2 = make_step(w, 1, base), make_step(w, 2, base)
    assert np.array_equal(s1["k"], s2["k"]) and not np.array_equal(s1["q"], s2["q"])
    assert abs(float((s1["q"] - base["q"]).std()) - 0.05) < 0.005


def test_columns_pattern_plants_shared_stripes():
    w = scaled(WORKLOADS["pulsecol_dream7b_16k"], seq_len=1024, q_heads=8, kv_heads=2, n_stripe_columns=16)
    x = make_base(w)
    # a stripe key has a much larger norm than a plain N(0,1) key of d=128 ... on average over stripes
    norms = np.linalg.norm(x["k"][0, 0], axis=-1)
    assert (norms > np.sqrt(128) + 1.5).sum() >= 8


def test_planting_follows_the_kv_groups():
    """Every pattern builds on a GQA shape with a ragged length, and the query heads of one
    kv group receive the same planted shift (the shift of their kv head's pattern)."""
    for name, extra in (("sparsed_64k", 0.02), ("pulsecol_dream7b_16k", 0.0)):
        w = scaled(WORKLOADS[name], seq_len=1000, q_heads=8, kv_heads=2, extra_pair_frac=extra,
                   n_stripe_columns=16)
        planted = make_base(w)
        plain = make_base(scaled(w, pattern="plain", extra_pair_frac=0.0))
        np.testing.assert_array_equal(planted["v"], plain["v"])
        dq = planted["q"] - plain["q"]
        assert np.linalg.norm(planted["k"] - plain["k"], axis=-1).max() > 1.0
        for g in range(2):
            grp = dq[:, 4 * g:4 * (g + 1)]
            assert np.linalg.norm(grp, axis=-1).max() > 1.0
            # (q + shift) - q is the shift up to fp32 rounding of the sum
            np.testing.assert_allclose(grp, np.broadcast_to(grp[:, :1], grp.shape), rtol=0, atol=1e-5)
        assert not np.array_equal(dq[:, 0], dq[:, 4])
    # the smoke test's shape: four query heads over two kv heads, three steps after the base
    w = scaled(WORKLOADS["sparsed_64k"], seq_len=1000, q_heads=4, kv_heads=2, total_steps=4, dense_steps=1,
               select_step=1, keep_frac=0.25)
    base = make_base(w)
    for t in range(w.total_steps):
        x = make_step(w, t, base)
        assert x["q"].shape == (1, 4, 1000, 128) and x["k"].shape == (1, 2, 1000, 128)


def _cov(T, s, t):
    from workloads.generate import walk_nodes
    cs, ct = dict(walk_nodes(T, s)), dict(walk_nodes(T, t))
    return sum(c * ct.get(k, 0.0) for k, c in cs.items())


def test_walk_has_the_covariance_of_a_unit_step_random_walk():
    """Cov(W_s, W_t) = min(s, t) for every pair of steps, exactly (the node
    draws are independent standard normals): W_0 = 0 and the increments are
    independent with unit variance.  Checked over whole schedules, including
    lengths that are not powers of two."""
    for T in (1, 4, 7, 32, 192):
        for s in range(T + 1):
            for t in range(s, T + 1):
                assert abs(_cov(T, s, t) - s) < 1e-9, (T, s, t)
    for s, t in ((204, 205), (205, 1023), (0, 1023), (511, 512), (1023, 1024)):
        assert abs(_cov(1024, s, t) - min(s, t)) < 1e-9


def test_walk_steps_drift_by_sigma_per_step():
    """Generated tensors: consecutive steps differ by sigma N(0, 1) per element,
    successive increments are uncorrelated, and V stays fixed."""
    w = scaled(WORKLOADS["llada8b_8k"], seq_len=2048, q_heads=4, kv_heads=4, dtype="f32", total_steps=64)
    base = make_base(w)
    xs = [make_step(w, t, base) for t in (30, 31, 32, 33)]
    for n in "qk":
        d1 = (xs[1][n] - xs[0][n]).astype(np.float64).ravel()
        d2 = (xs[2][n] - xs[1][n]).astype(np.float64).ravel()
        d3 = (xs[3][n] - xs[2][n]).astype(np.float64).ravel()
        for d in (d1, d2, d3):
            assert abs(d.std() / w.step_sigma - 1.0) < 0.01 and abs(d.mean()) < 0.01 * w.step_sigma
        for a, b in ((d1, d2), (d2, d3)):
            assert abs(np.corrcoef(a, b)[0, 1]) < 0.01
        drift = (xs[3][n] - base[n]).astype(np.float64).ravel()
        assert abs(drift.std() / (w.step_sigma * np.sqrt(33)) - 1.0) < 0.01
    np.testing.assert_array_equal(xs[0]["v"], xs[3]["v"])


def test_walk_does_not_depend_on_the_thread_pool(monkeypatch):
    w = scaled(WORKLOADS["sparsed_64k"], seq_len=4096, q_heads=2, kv_heads=2, total_steps=1024)
    base = make_base(w)
    a = make_step(w, 205, base)
    monkeypatch.setattr("os.cpu_count", lambda: 1)
    b = make_step(w, 205, base)
    for n in "qkv":
        assert _h(a[n]) == _h(b[n])
