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
    counts = {a: acts.count(a) for a in gold["counts"]}
    assert counts == gold["counts"] and sum(counts.values()) == len(acts)  # no probes in these schedules
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


# ---- adaptive anchors: probes, pattern overlap, adoption ----------------------

def _random_csr(rng, rows, nkb, density):
    """Random CSR pattern (ascending rows, some empty) and its dense boolean mask."""
    dense = rng.random((rows, nkb)) < density
    rp = np.zeros(rows + 1, dtype=np.int32)
    rp[1:] = np.cumsum(dense.sum(1))
    ci = np.nonzero(dense)[1].astype(np.int32)  # row-major order: ascending within a row
    return rp, ci, dense


def test_probe_actions_hand_listed():
    # T=10, warm-up 2, selection at 2, refresh every 4 (S = {2, 6}), probes every 3
    acts = oracle.schedule_actions(10, 2, 2, 4, (), False, probe_interval=3)
    assert acts == ["DENSE", "DENSE", "SELECT_SPARSE", "SPARSE", "SPARSE", "PROBE_SPARSE", "SELECT_SPARSE",
                    "SPARSE", "PROBE_SPARSE", "SPARSE"]
    # no probe inside the warm-up or at the selection step itself
    acts = oracle.schedule_actions(8, 4, 1, 0, (), False, probe_interval=1)
    assert acts == ["DENSE", "DENSE_SELECT", "DENSE", "DENSE"] + ["PROBE_SPARSE"] * 4
    assert oracle.schedule_actions(6, 1, 0, probe_interval=0) == ["DENSE_SELECT"] + ["SPARSE"] * 5


@pytest.mark.parametrize("seed", range(6))
def test_mask_overlap_equals_dense_boolean_counts(seed):
    """|A n B|, |A|, |B| of the set form against boolean masks (brute force)."""
    rng = np.random.default_rng(seed)
    rows, nkb = int(rng.integers(1, 40)), int(rng.integers(1, 20))
    ra, ca, da = _random_csr(rng, rows, nkb, rng.uniform(0, 1))
    rb, cb, db = _random_csr(rng, rows, nkb, rng.uniform(0, 1))
    assert oracle.mask_overlap(ra, ca, rb, cb) == (int((da & db).sum()), int(da.sum()), int(db.sum()))


def test_mask_overlap_closed_forms():
    rng = np.random.default_rng(7)
    rp, ci, d = _random_csr(rng, 12, 9, 0.4)
    n = int(d.sum())
    assert oracle.mask_overlap(rp, ci, rp, ci) == (n, n, n)  # identical
    rc, cc, dc = _random_csr(np.random.default_rng(0), 12, 9, 0.0)
    # complement of a pattern: disjoint, union is every (row, block) pair
    comp = ~d
    rq = np.zeros(13, dtype=np.int32)
    rq[1:] = np.cumsum(comp.sum(1))
    cq = np.nonzero(comp)[1].astype(np.int32)
    inter, na, nb = oracle.mask_overlap(rp, ci, rq, cq)
    assert inter == 0 and na + nb == 12 * 9
    assert oracle.mask_overlap(rp, ci, rc, cc) == (0, n, 0)  # against the empty pattern
    # the same blocks in different rows do not overlap
    a = (np.array([0, 1, 1]), np.array([3]))
    b = (np.array([0, 0, 1]), np.array([3]))
    assert oracle.mask_overlap(*a, *b) == (0, 1, 1)


def test_overlap_ratio_and_adoption_rule():
    # A = {(0,1), (0,2)}, B = {(0,2), (0,3)}: one shared pair of three
    inter, na, nb = oracle.mask_overlap(np.array([0, 2]), np.array([1, 2]), np.array([0, 2]), np.array([2, 3]))
    assert (inter, na, nb) == (1, 2, 2)
    assert oracle.overlap_ratio(inter, na, nb) == 1 / 3
    assert oracle.overlap_ratio(0, 0, 0) == 1.0  # both empty: identical
    assert oracle.overlap_ratio(0, 3, 0) == 0.0
    assert oracle.overlap_ratio(5, 5, 5) == 1.0
    # strict: J equal to the threshold keeps the cached pattern
    assert not oracle.probe_adopts(1, 2, 2, 1 / 3)
    assert oracle.probe_adopts(1, 2, 2, 0.34)
    assert not oracle.probe_adopts(5, 5, 5, 1.0)  # identical patterns are never replaced
    assert oracle.probe_adopts(4, 5, 5, 1.0)
    assert not oracle.probe_adopts(0, 5, 5, 0.0)  # threshold 0: never adopt


def test_probe_schedule_keeps_a_stable_pattern_and_adopts_a_moved_one():
    """Tiny fp32 schedule with probes: inputs that barely change keep the
    step-0 pattern; at step 4 the inputs are replaced by unrelated ones, the
    probe's overlap drops and it is adopted, and step 5 attends with it."""
    w = scaled(WORKLOADS["tiny_fp32_h4_l512"], total_steps=6, probe_interval=2, min_overlap=0.5)
    base = make_base(w)
    other = make_base(scaled(w, wid=101))

    def inputs(t):
        return make_step(w, t, base if t < 4 else other)

    res = oracle.run_schedule(w, inputs)
    assert [r["action"] for r in res] == ["DENSE_SELECT", "SPARSE", "PROBE_SPARSE", "SPARSE", "PROBE_SPARSE",
                                          "SPARSE"]
    p2, p4 = res[2]["probe"], res[4]["probe"]
    assert not p2["adopted"] and oracle.overlap_ratio(*p2["counts"]) >= 0.5
    assert p4["adopted"] and oracle.overlap_ratio(*p4["counts"]) < 0.5
    assert res[2]["pattern"] is res[0]["pattern"] and res[3]["pattern"] is res[0]["pattern"]
    # the adopted pattern is the selection on step 4's inputs
    x4 = inputs(4)
    rp, ci = oracle.select_topk(oracle.pooled_mass(x4["q"], x4["k"], 64, 64), 0.25)
    np.testing.assert_array_equal(res[4]["pattern"][0], rp)
    np.testing.assert_array_equal(res[4]["pattern"][1], ci)
    x5 = inputs(5)
    o, lse = oracle.block_sparse_attention(x5["q"], x5["k"], x5["v"], rp, ci, 64, 64)
    np.testing.assert_allclose(res[5]["o"], o, atol=0)


def test_exact_selector_schedule_selects_after_the_dense_pass():
    """Exact block mass: the selection step runs dense attention, its lse gives
    the mass, and the pattern applies from the next step."""
    w = scaled(WORKLOADS["tiny_fp32_h4_l512"], selector="blocks_exact", refresh_dense=True, total_steps=5,
               dense_steps=2, select_step=1, refresh_interval=2)
    base = make_base(w)
    res = oracle.run_schedule(w, lambda t: make_step(w, t, base))
    assert [r["action"] for r in res] == ["DENSE", "DENSE_SELECT", "SPARSE", "DENSE_SELECT", "SPARSE"]
    x1 = make_step(w, 1, base)
    o1, lse1 = oracle.dense_attention(x1["q"], x1["k"], x1["v"])
    np.testing.assert_allclose(res[1]["o"], o1, atol=0)
    rp, ci = oracle.select_topk(oracle.exact_block_mass(x1["q"], x1["k"], lse1, 64, 64), 0.25)
    np.testing.assert_array_equal(res[1]["pattern"][0], rp)
    np.testing.assert_array_equal(res[1]["pattern"][1], ci)
    x2 = make_step(w, 2, base)
    o2, _ = oracle.block_sparse_attention(x2["q"], x2["k"], x2["v"], rp, ci, 64, 64)
    np.testing.assert_allclose(res[2]["o"], o2, atol=0)
    # the planted sink is found by the exact mass too
    assert np.all((ci.reshape(4, 8, 2)[0] == 0).any(-1))
