"""Pins of the LoSA-style oracle (oracle/losa.py) to things other than itself:
closed forms of the locality score, brute-force orderings in plain Python, set
unions, a planted page the selector must find, and torch's fused attention
with a boolean mask for the attention over (union pages + block).  The last
tests plant one mistake at a time in the oracle and check that a pin fails."""

import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.losa as olosa
from workloads import tiny_random
from workloads.configs import LOSA_WORKLOADS, scaled
from workloads.generate import make_losa_base, make_losa_cache, make_losa_iteration


def _blk(seed, B=1, Hq=4, Hkv=2, Lp=48, Bs=6, d=8):
    """Tiny block-wise inputs in float64: prefix caches and a block."""
    pre = tiny_random(seed, B, Hq, Hkv, Lp, d)
    blk = tiny_random(seed + 500, B, Hq, Hkv, Bs, d)
    prev = tiny_random(seed + 900, B, Hq, Hkv, Bs, d)
    f = lambda a: a.astype(np.float64)
    return {"q": f(blk["q"]), "q_prev": f(prev["q"]), "k_cache": f(pre["k"]), "v_cache": f(pre["v"]),
            "k_blk": f(blk["k"]), "v_blk": f(blk["v"])}


# ---------------------------------------------------------------- pins

def pin_locality_closed_forms():
    x = _blk(1)
    q = x["q"]
    assert np.all(olosa.locality_scores(q, q) == 0.0)
    np.testing.assert_allclose(olosa.locality_scores(q + 0.75, q), 0.5625, rtol=1e-14)
    # one channel of one head of token 2 moves by 3: delta_2 = 9 / (Hq d)
    q2 = q.copy()
    q2[0, 3, 2, 5] += 3.0
    want = np.zeros((1, 6))
    want[0, 2] = 9.0 / (4 * 8)
    np.testing.assert_allclose(olosa.locality_scores(q2, q), want, atol=1e-13)


def pin_active_brute_force():
    delta = np.array([[0.5, 2.0, 0.5, 3.0, 2.0, 0.1, 2.0]])
    for n in range(1, 8):
        want = sorted(sorted(range(7), key=lambda i: (-delta[0, i], i))[:n])
        assert list(olosa.select_active(delta, n)[0]) == want
    assert list(olosa.select_active(np.zeros((1, 5)), 3)[0]) == [0, 1, 2]  # ties: lowest indices


def pin_page_pooling():
    x = _blk(2)
    kp = olosa.pool_pages(x["k_cache"], 16)
    np.testing.assert_allclose(kp.sum(axis=2) * 16, x["k_cache"].sum(axis=2), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(olosa.pool_pages(x["k_cache"], 1), x["k_cache"])


def pin_planted_page():
    """Kv head 1 holds zero keys except page 2, every key of which is c * q of
    query head 3, token 4; head 3 must score that page scale * c * |q|^2 and
    keep it first; heads 0, 1 (kv head 0) must not see it."""
    x = _blk(3)
    kc = np.zeros_like(x["k_cache"])
    c = 0.5
    kc[0, 1, 2 * 8:3 * 8] = c * x["q"][0, 3, 4]
    kp = olosa.pool_pages(kc, 8)
    active = np.array([[1, 4]])
    s = olosa.page_scores(x["q"], active, kp)
    np.testing.assert_allclose(s[0, 3, 1, 2], c * np.dot(x["q"][0, 3, 4], x["q"][0, 3, 4]) / math.sqrt(8), rtol=1e-13)
    assert np.all(s[0, :2] == 0.0)
    sel = olosa.select_pages(s, 1)
    assert sel[0, 3, 1, 0] == 2


def pin_page_select_brute_force():
    r = np.random.default_rng(4)
    s = np.round(r.standard_normal((1, 2, 3, 9)), 1)  # rounding makes ties
    for k in (1, 3, 9):
        sel = olosa.select_pages(s, k)
        for h, a in itertools.product(range(2), range(3)):
            row = s[0, h, a]
            want = sorted(sorted(range(9), key=lambda P: (-row[P], P))[:k])
            assert list(sel[0, h, a]) == want


def pin_union_sets():
    r = np.random.default_rng(5)
    sel = np.sort(np.stack([[r.choice(20, 4, replace=False) for _ in range(3)] for _ in range(6)])[None], axis=-1)
    un = olosa.union_pages(sel, 2)  # Hq=6, Hkv=2: heads 0-2 -> 0, 3-5 -> 1
    for g in range(2):
        want = sorted(set().union(*[set(sel[0, h, a]) for h in range(3 * g, 3 * g + 3) for a in range(3)]))
        assert list(un[0][g]) == want


def _sdpa_masked(q, k, v, allowed):
    """torch's fused attention with a boolean mask, kv heads repeated per group."""
    G = q.shape[1] // k.shape[1]
    kt = torch.from_numpy(np.repeat(k, G, axis=1))
    vt = torch.from_numpy(np.repeat(v, G, axis=1))
    m = torch.from_numpy(np.repeat(allowed, G, axis=1))
    return torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), kt, vt, attn_mask=m).numpy()


def pin_dense_vs_sdpa():
    x = _blk(6)
    o, lse = olosa.losa_dense(x["q"], x["k_cache"], x["v_cache"], x["k_blk"], x["v_blk"])
    k = np.concatenate([x["k_cache"], x["k_blk"]], axis=2)
    v = np.concatenate([x["v_cache"], x["v_blk"]], axis=2)
    ref = _sdpa_masked(x["q"], k, v, np.ones((1, 2, 6, 54), dtype=bool))
    np.testing.assert_allclose(o, ref, atol=1e-12)
    s = np.einsum("bhid,bhjd->bhij", x["q"], np.repeat(k, 2, axis=1)) / math.sqrt(8)
    m = s.max(-1)
    np.testing.assert_allclose(lse, m + np.log(np.exp(s - m[..., None]).sum(-1)), atol=1e-12)


def pin_partial_vs_sdpa_and_brute_force():
    """Active rows against torch's masked attention (prefix tokens of the
    union + all block keys) and against a loop over the keys with math.fsum;
    Stable rows keep their previous values bit for bit."""
    x = _blk(7)
    page = 8
    active = np.array([[0, 3, 5]])
    unions = [[np.array([1, 4]), np.array([0, 2, 5])]]
    o_prev = np.full((1, 4, 6, 8), 7.25)
    lse_prev = np.full((1, 4, 6), -3.5)
    o, lse = olosa.losa_attention(x["q"], x["k_cache"], x["v_cache"], x["k_blk"], x["v_blk"], active, unions, page,
                                  o_prev, lse_prev)
    allowed = np.zeros((1, 2, 6, 54), dtype=bool)
    allowed[..., 48:] = True
    for g, u in enumerate(unions[0]):
        for P in u:
            allowed[0, g, :, P * page:(P + 1) * page] = True
    k = np.concatenate([x["k_cache"], x["k_blk"]], axis=2)
    v = np.concatenate([x["v_cache"], x["v_blk"]], axis=2)
    ref = _sdpa_masked(x["q"], k, v, allowed)
    np.testing.assert_allclose(o[:, :, active[0]], ref[:, :, active[0]], atol=1e-12)
    stable = [i for i in range(6) if i not in active[0]]
    assert np.all(o[:, :, stable] == 7.25) and np.all(lse[:, :, stable] == -3.5)
    # brute force, one row: exp of every allowed score, no max subtracted
    h, i = 2, 3
    g = 1
    keys = [j for j in range(54) if allowed[0, g, 0, j]]
    w = [math.exp(sum(x["q"][0, h, i, c] * k[0, g, j, c] for c in range(8)) / math.sqrt(8)) for j in keys]
    l = math.fsum(w)
    for c in range(8):
        assert abs(o[0, h, i, c] - math.fsum(wj * v[0, g, j, c] for wj, j in zip(w, keys)) / l) < 1e-12
    assert abs(lse[0, h, i] - math.log(l)) < 1e-12


def pin_full_union_is_dense():
    x = _blk(8)
    page = 8
    full = [[np.arange(6), np.arange(6)]]
    o_prev = np.zeros((1, 4, 6, 8))
    o, lse = olosa.losa_attention(x["q"], x["k_cache"], x["v_cache"], x["k_blk"], x["v_blk"],
                                  np.arange(6)[None], full, page, o_prev, np.zeros((1, 4, 6)))
    od, ld = olosa.losa_dense(x["q"], x["k_cache"], x["v_cache"], x["k_blk"], x["v_blk"])
    np.testing.assert_allclose(o, od, atol=1e-13)
    np.testing.assert_allclose(lse, ld, atol=1e-13)


def pin_moving_tokens_are_active():
    """On the block-wise generator, the tokens given the large change at an
    iteration are exactly the Active ones when n_active equals their count."""
    w = scaled(LOSA_WORKLOADS["losa_sdar8b_32k"], q_heads=4, kv_heads=2, prefix_len=256, block_len=16, head_dim=16,
               page=16, pages_per_query=2, n_active=5, n_moving=5, dtype="f32")
    base = make_losa_base(w)
    for t in (1, 2, 5):
        q1 = make_losa_iteration(w, t, base)["q"].astype(np.float64)
        q0 = make_losa_iteration(w, t - 1, base)["q"].astype(np.float64)
        moved = np.sort(np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.wid, 1 + t, 9]))).choice(
            16, size=5, replace=False))
        assert list(olosa.select_active(olosa.locality_scores(q1, q0), 5)[0]) == list(moved)


PINS = [pin_locality_closed_forms, pin_active_brute_force, pin_page_pooling, pin_planted_page,
        pin_page_select_brute_force, pin_union_sets, pin_dense_vs_sdpa, pin_partial_vs_sdpa_and_brute_force,
        pin_full_union_is_dense, pin_moving_tokens_are_active]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_losa_pin(pin):
    pin()


def test_losa_step_composes_the_pieces():
    """losa_step on the small block-wise workload: unions hold every row's
    selection, stay within G * n_active * k pages, and are ascending."""
    w = scaled(LOSA_WORKLOADS["losa_sdar8b_32k"], q_heads=4, kv_heads=2, prefix_len=512, block_len=16, head_dim=16,
               page=16, pages_per_query=3, n_active=4)
    base = make_losa_base(w)
    cache = make_losa_cache(w, base)
    x0, x1 = make_losa_iteration(w, 0, base), make_losa_iteration(w, 1, base)
    o0, l0 = olosa.losa_dense(x0["q"], cache["k_cache"], cache["v_cache"], x0["k_blk"], x0["v_blk"])
    r = olosa.losa_step(x1["q"], x0["q"], cache["k_cache"], cache["v_cache"], x1["k_blk"], x1["v_blk"], o0, l0,
                        w.page, w.n_active, w.pages_per_query)
    for g in range(2):
        u = r["unions"][0][g]
        assert np.all(np.diff(u) > 0) and len(u) <= 2 * 4 * 3
        for h in (2 * g, 2 * g + 1):
            assert set(r["sel"][0, h].ravel()) <= set(u)
    assert r["o"].shape == o0.shape and np.isfinite(r["lse"]).all()


# ---------------------------------------------------------------- planted mistakes

def _mutants():
    def loc_abs(q, q_prev):
        dq = oracle.attention.as_f64(q) - oracle.attention.as_f64(q_prev)
        B, Hq, Bs, d = dq.shape
        return np.abs(dq).transpose(0, 2, 1, 3).reshape(B, Bs, Hq * d).mean(axis=-1)

    def loc_per_head0(q, q_prev):  # only the first head's change
        dq = oracle.attention.as_f64(q)[:, :1] - oracle.attention.as_f64(q_prev)[:, :1]
        return (dq * dq).mean(axis=(1, 3))

    def active_smallest(delta, n):
        return np.sort(np.argsort(np.asarray(delta), axis=1, kind="stable")[:, :n], axis=1)

    def scores_pooled_group(q, active, kp, scale=None):  # wrong head -> kv head map (h % Hkv)
        q, kp = oracle.attention.as_f64(q), np.asarray(kp)
        B, Hq, Bs, d = q.shape
        s = np.zeros((B, Hq, active.shape[1], kp.shape[2]))
        for h in range(Hq):
            s[0, h] = (q[0, h, active[0]] @ kp[0, h % kp.shape[1]].T) / math.sqrt(d)
        return s

    def select_pages_unsorted_ties(scores, k):  # ties broken towards the higher page
        B, Hq, n_a, npg = scores.shape
        out = np.zeros((B, Hq, n_a, k), dtype=np.int64)
        for b, h, a in itertools.product(range(B), range(Hq), range(n_a)):
            out[b, h, a] = np.sort(np.lexsort((-np.arange(npg), -scores[b, h, a]))[:k])
        return out

    def union_per_head(sel, kv_heads):  # the first head of the group only
        B, Hq = sel.shape[:2]
        G = Hq // kv_heads
        return [[np.unique(sel[b, g * G].ravel()) for g in range(kv_heads)] for b in range(B)]

    def block_attention_no_block(q, k_cache, v_cache, k_blk, v_blk, allowed_prefix, rows, scale=None):
        # the suffix contribution dropped: only the union tokens of the prefix
        Bs = q.shape[2]
        big = np.concatenate([allowed_prefix, np.zeros(allowed_prefix.shape[:2] + (Bs,), dtype=bool)], axis=2)
        qq = oracle.attention.as_f64(q)
        k, v = olosa._concat_keys(k_cache, v_cache, k_blk, v_blk)
        grp = oracle.head_group(qq.shape[1], k.shape[1])
        o = np.zeros((qq.shape[0], qq.shape[1], rows.shape[1], v.shape[-1]))
        lse = np.zeros(o.shape[:3])
        for b in range(qq.shape[0]):
            for h in range(qq.shape[1]):
                s = (qq[b, h, rows[b]] @ k[b, grp[h]].T) / math.sqrt(qq.shape[-1])
                s = np.where(big[b, grp[h]][None, :], s, -np.inf)
                o[b, h], lse[b, h] = oracle.attention._attend(s, v[b, grp[h]])
        return o, lse

    def union_mask_off_by_one(unions, Lp, page):
        m = np.zeros((len(unions), len(unions[0]), Lp), dtype=bool)
        for b, per in enumerate(unions):
            for g, u in enumerate(per):
                for P in u:
                    m[b, g, P * page + 1:(P + 1) * page + 1] = True
        return m

    return [
        ("locality_scores", loc_abs),
        ("locality_scores", loc_per_head0),
        ("select_active", active_smallest),
        ("page_scores", scores_pooled_group),
        ("select_pages", select_pages_unsorted_ties),
        ("union_pages", union_per_head),
        ("block_attention", block_attention_no_block),
        ("union_token_mask", union_mask_off_by_one),
    ]


@pytest.mark.parametrize("name,impl", _mutants(), ids=lambda v: v if isinstance(v, str) else v.__name__)
def test_losa_mutant_is_caught(monkeypatch, name, impl):
    monkeypatch.setattr(olosa, name, impl)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake in {name} ({impl.__name__})"
