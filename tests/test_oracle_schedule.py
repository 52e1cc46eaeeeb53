"""Pins of the oracle's step schedule and of the whole-schedule runner (CPU)."""

import json
import os

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, make_base, make_step
from workloads.configs import scaled

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "schedule_counts.json")


def _acts(w):
    return oracle.schedule_actions(w.total_steps, w.dense_steps, w.select_step, w.refresh_interval,
                                   w.refresh_steps, w.refresh_dense)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_action_counts_match_hand_counts(name):
    gold = json.load(open(GOLDEN))[name]
    acts = _acts(WORKLOADS[name])
    counts = {a: acts.count(a) for a in oracle.ACTIONS}
    assert counts == gold["counts"]
    sel = [t for t, a in enumerate(acts) if a in ("DENSE_SELECT", "SELECT_SPARSE")]
    if "select_steps" in gold:
        assert sel == gold["select_steps"]
    assert acts.index("SPARSE") == gold["first_sparse"] or acts[gold["first_sparse"]] == "SELECT_SPARSE"


def test_sparse_never_precedes_a_pattern():
    with pytest.raises(ValueError):
        oracle.schedule_actions(10, 2, 5)


def test_tiny_schedule_reuses_step0_mask_and_equals_masked_definition():
    w = WORKLOADS["tiny_fp32_h4_l512"]
    base = make_base(w)
    res = oracle.run_schedule(w, lambda t: make_step(w, t, base))
    assert [r["action"] for r in res] == ["DENSE_SELECT", "SPARSE", "SPARSE", "SPARSE"]
    rp, ci = res[0]["pattern"]
    assert all(r["pattern"] is res[0]["pattern"] for r in res)  # computed once, reused
    assert len(ci) == 4 * 8 * 2 and np.all(np.diff(rp) == 2)
    # a sparse step equals dense attention with -inf outside the kept blocks
    x = make_step(w, 2, base)
    allowed = oracle.block_token_mask(rp, ci, 1, 4, 512, 64, 64)
    o, lse = oracle.masked_attention(x["q"], x["k"], x["v"], allowed)
    np.testing.assert_allclose(res[2]["o"], o, atol=1e-12)
    np.testing.assert_allclose(res[2]["lse"], lse, atol=1e-12)


def test_planted_structure_is_found_by_the_selector():
    """The sink head keeps key block 0 in every row; the local head keeps
    blocks inside its +-2 band (sanity of the generator + selector, not parity)."""
    w = WORKLOADS["tiny_fp32_h4_l512"]
    x = make_step(w, 0)
    A = oracle.pooled_mass(x["q"], x["k"], 64, 64)
    rp, ci = oracle.select_topk(A, 0.25)
    rows = ci.reshape(4, 8, 2)
    assert np.all((rows[0] == 0).any(-1))
    assert np.all(np.abs(rows[1] - np.arange(8)[:, None]) <= 2)


def test_column_schedule_on_a_small_gqa_case():
    w = scaled(WORKLOADS["pulsecol_dream7b_16k"], q_heads=4, kv_heads=2, seq_len=256, head_dim=16,
               total_steps=6, refresh_steps=(3,), n_stripe_columns=8, column_keep_frac=0.05)
    base = make_base(w)
    res = oracle.run_schedule(w, lambda t: make_step(w, t, base, as_float=True))
    assert [r["action"] for r in res] == ["DENSE_SELECT", "SPARSE", "SPARSE", "DENSE_SELECT", "SPARSE", "SPARSE"]
    cols0, cols3 = res[1]["pattern"], res[4]["pattern"]
    assert cols0.shape == (1, 2, 13)
    x = make_step(w, 4, base, as_float=True)
    o, lse = oracle.column_sparse_attention(x["q"], x["k"], x["v"], cols3)
    np.testing.assert_allclose(res[4]["o"], o, atol=0)
