"""The pins catch plausible mistakes: each test plants one mistake in the
oracle (on the CPU, through monkeypatch) and checks that a pin now fails."""

import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
import oracle.attention as oatt
import oracle.schedule as osch
import oracle.select as osel
from workloads import tiny_random


def _x(seed, Hq=4, Hkv=2, L=13, d=8):
    return {n: v.astype(np.float64) for n, v in tiny_random(seed, 1, Hq, Hkv, L, d).items()}


def pin_dense_vs_torch():
    x = _x(1)
    o, lse = oracle.dense_attention(x["q"], x["k"], x["v"])
    kt = torch.from_numpy(np.repeat(x["k"], 2, axis=1))
    vt = torch.from_numpy(np.repeat(x["v"], 2, axis=1))
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(x["q"]), kt, vt).numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)
    s = np.einsum("bhid,bhjd->bhij", x["q"], kt.numpy()) / np.sqrt(8)
    np.testing.assert_allclose(lse, logsumexp(s, axis=-1), atol=1e-12)


def pin_pooling_closed_form():
    x = np.arange(5, dtype=np.float64).reshape(1, 1, 5, 1)
    np.testing.assert_array_equal(oracle.pool_blocks(x, 2)[0, 0, :, 0], [0.5, 2.5, 4.0])


def pin_topk_ties_brute_force():
    A = np.array([[[[1.0, 3.0, 2.0, 3.0, 0.0, 2.0]]]])
    rp, ci = oracle.select_topk(A, 0.5)
    best = min(itertools.combinations(range(6), 3), key=lambda S: (-sum(A[0, 0, 0, list(S)]), S))
    assert list(ci) == list(best)


def pin_mass_exact_hit():
    # cumulative masses 0.5, 0.75, 0.875, 1: tau = 0.75 is reached by 2 blocks
    A = np.array([[[[0.125, 0.5, 0.25, 0.125]]]])
    rp, ci, _ = oracle.select_mass_cap(A, 0.75, 1.0)
    assert list(ci) == [1, 2]


def pin_column_sum_total():
    x = _x(3, Hq=6, Hkv=2)
    _, lse = oracle.dense_attention(x["q"], x["k"], x["v"])
    C = oracle.column_scores(x["q"], x["k"], lse)
    np.testing.assert_allclose(C.sum(-1), 3 * 13, rtol=1e-12)


def pin_topk_count():
    A = np.random.default_rng(0).random((1, 1, 2, 256))
    rp, _ = oracle.select_topk(A, 0.10)
    assert np.all(np.diff(rp) == 26)


def pin_overlap_rows_matter():
    # block 3 kept in row 0 of A and in row 1 of B: no common (row, block) pair
    assert oracle.mask_overlap(np.array([0, 1, 1]), np.array([3]), np.array([0, 0, 1]), np.array([3])) == (0, 1, 1)


def pin_overlap_ratio_hand():
    # A = {(0,1), (0,2)}, B = {(0,2), (0,3)}: J = 1/3
    c = oracle.mask_overlap(np.array([0, 2]), np.array([1, 2]), np.array([0, 2]), np.array([2, 3]))
    assert oracle.overlap_ratio(*c) == 1 / 3


def pin_adoption_strict():
    assert not oracle.probe_adopts(1, 2, 2, 1 / 3) and oracle.probe_adopts(1, 2, 2, 0.34)


def pin_probe_steps_hand():
    assert oracle.schedule_actions(10, 2, 2, 4, (), False, probe_interval=3)[5] == "PROBE_SPARSE"
    assert oracle.schedule_actions(10, 2, 2, 4, (), False, probe_interval=3).count("PROBE_SPARSE") == 2


def test_pins_pass_on_the_real_oracle():
    for pin in (pin_dense_vs_torch, pin_pooling_closed_form, pin_topk_ties_brute_force,
                pin_mass_exact_hit, pin_column_sum_total, pin_topk_count, pin_overlap_rows_matter,
                pin_overlap_ratio_hand, pin_adoption_strict, pin_probe_steps_hand, pin_exact_mass_rows):
        pin()


def _fails(pin):
    with pytest.raises(AssertionError):
        pin()


def test_transposed_gqa_map_is_caught(monkeypatch):
    bad = lambda hq, hkv: np.arange(hq) % hkv  # noqa: E731  interleaved instead of consecutive groups
    monkeypatch.setattr(oatt, "head_group", bad)
    _fails(pin_dense_vs_torch)


def test_dropped_scale_is_caught(monkeypatch):
    monkeypatch.setattr(oatt, "default_scale", lambda d: 1.0)
    _fails(pin_dense_vs_torch)


def test_lse_sign_error_is_caught(monkeypatch):
    real = oatt._attend

    def bad(s, v):
        o, lse = real(s, v)
        m = s.max(axis=-1)
        return o, m - (lse - m)
    monkeypatch.setattr(oatt, "_attend", bad)
    _fails(pin_dense_vs_torch)


def test_value_operand_transposed_is_caught(monkeypatch):
    real = oatt._attend
    monkeypatch.setattr(oatt, "_attend", lambda s, v: real(s.T.copy() if s.shape[0] == s.shape[1] else s, v))
    _fails(pin_dense_vs_torch)


def test_pooling_off_by_one_is_caught(monkeypatch):
    def bad(x, block):
        x = oatt.as_f64(x)
        B, H, L, d = x.shape
        nb = -(-L // block)
        out = np.zeros((B, H, nb, d))
        for I in range(nb):
            seg = x[:, :, I * block + 1:min(L, (I + 1) * block + 1)]
            out[:, :, I] = seg.sum(axis=2) / max(1, seg.shape[2])
        return out
    monkeypatch.setattr(osel, "pool_blocks", bad)
    monkeypatch.setattr(oracle, "pool_blocks", bad)
    _fails(pin_pooling_closed_form)


def test_tie_break_toward_higher_index_is_caught(monkeypatch):
    monkeypatch.setattr(osel, "rank_order", lambda a: np.lexsort((-np.arange(len(a)), -np.asarray(a))))
    _fails(pin_topk_ties_brute_force)


def test_strict_mass_comparison_is_caught(monkeypatch):
    def bad(A, tau):
        n = A.shape[-1]
        out = []
        for a in A.reshape(-1, n):
            c = np.cumsum(a[osel.rank_order(a)])
            hit = np.nonzero(c > tau)[0]
            out.append(hit[0] + 1 if len(hit) else n)
        return np.array(out)
    monkeypatch.setattr(osel, "mass_prefix_counts", bad)
    _fails(pin_mass_exact_hit)


def test_missing_group_head_in_column_scores_is_caught(monkeypatch):
    real = osel.head_group
    monkeypatch.setattr(osel, "head_group", lambda hq, hkv: np.where(np.arange(hq) % (hq // hkv) == 0, -10**6,
                                                                     real(hq, hkv)))
    with pytest.raises((AssertionError, IndexError)):
        pin_column_sum_total()


def test_floor_instead_of_ceil_count_is_caught(monkeypatch):
    monkeypatch.setattr(osel, "count_from_fraction",
                        lambda f, n: max(1, int(Fraction(str(f)) * n)))
    _fails(pin_topk_count)


def test_overlap_that_ignores_rows_is_caught(monkeypatch):
    monkeypatch.setattr(osch, "_pairs", lambda rp, ci: {int(c) for c in np.asarray(ci)})
    _fails(pin_overlap_rows_matter)


def test_union_taken_as_the_larger_pattern_is_caught(monkeypatch):
    monkeypatch.setattr(osch, "overlap_ratio", lambda i, a, b: 1.0 if max(a, b) == 0 else i / max(a, b))
    monkeypatch.setattr(oracle, "overlap_ratio", osch.overlap_ratio)
    _fails(pin_overlap_ratio_hand)


def test_adoption_at_equality_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "probe_adopts", lambda i, a, b, th: osch.overlap_ratio(i, a, b) <= th)
    _fails(pin_adoption_strict)


def test_probes_counted_from_step_zero_are_caught(monkeypatch):
    real = osch.schedule_actions

    def bad(total_steps, dense_steps, select_step, refresh_interval=0, refresh_steps=(), refresh_dense=False,
            probe_interval=0):
        acts = real(total_steps, dense_steps, select_step, refresh_interval, refresh_steps, refresh_dense)
        return ["PROBE_SPARSE" if a == "SPARSE" and probe_interval and t % probe_interval == 0 else a
                for t, a in enumerate(acts)]
    monkeypatch.setattr(oracle, "schedule_actions", bad)
    _fails(pin_probe_steps_hand)


def pin_exact_mass_rows():
    x = _x(5, L=13)
    _, lse = oracle.dense_attention(x["q"], x["k"], x["v"])
    A = oracle.exact_block_mass(x["q"], x["k"], lse, 4, 3)  # partial last blocks on both sides
    np.testing.assert_allclose(A.sum(-1), 1.0, atol=1e-12)


def test_exact_mass_divided_by_the_nominal_block_size_is_caught(monkeypatch):
    real = osel.exact_block_mass

    def bad(q, k, lse, bq, bk, scale=None):
        A = real(q, k, lse, bq, bk, scale)
        L = np.asarray(q).shape[2]
        n_last = L - (A.shape[2] - 1) * bq
        A[:, :, -1] *= n_last / bq  # sum over the last block divided by bq, not by its size
        return A
    monkeypatch.setattr(oracle, "exact_block_mass", bad)
    _fails(pin_exact_mass_rows)


def test_exact_mass_without_the_lse_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "exact_block_mass",
                        lambda q, k, lse, bq, bk, scale=None: osel.exact_block_mass(q, k, np.zeros_like(lse), bq, bk))
    _fails(pin_exact_mass_rows)
