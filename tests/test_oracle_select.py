"""Pins of the oracle's pattern selection (CPU only).

  * pooling: closed-form means, including a partial last block;
  * pooled mass with one-token blocks equals the dense attention
    probability matrix (torch SDPA with one-hot V);
  * top-k: brute force over every k-subset (largest total mass, then the
    lexicographically smallest set), exact counts, invariants;
  * mass + cap: brute force over subsets for the shortest prefix, an
    exhaustive search over every subset sum for tau*, invariants;
  * column scores: the column sums of all rows' probabilities total G * L;
    with one query head per group they are the column sums of the
    probability matrix (torch SDPA with one-hot V); brute-force column top-k.
"""

import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.select import mass_prefix_counts
from workloads import tiny_random


def _probs_sdpa(q, k):
    """Probability matrix of dense attention via torch with V = identity."""
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    kt = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=1))
    eye = torch.eye(L, dtype=torch.float64).expand(B, Hq, L, L)
    return torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), kt, eye).numpy()


def test_pool_blocks_closed_form_with_partial_block():
    x = np.arange(5, dtype=np.float64).reshape(1, 1, 5, 1) * np.ones((1, 1, 5, 3))
    p = oracle.pool_blocks(x, 2)
    np.testing.assert_array_equal(p[0, 0, :, 0], [0.5, 2.5, 4.0])
    p3 = oracle.pool_blocks(x, 3)
    np.testing.assert_array_equal(p3[0, 0, :, 1], [1.0, 3.5])


def test_pool_blocks_matches_numpy_mean():
    x = np.random.default_rng(0).standard_normal((2, 3, 64, 8))
    np.testing.assert_allclose(oracle.pool_blocks(x, 16), x.reshape(2, 3, 4, 16, 8).mean(axis=3), atol=1e-15)


def test_pooled_mass_block1_equals_attention_probabilities():
    x = {n: v.astype(np.float64) for n, v in tiny_random(20, 1, 4, 2, 13, 8).items()}
    A = oracle.pooled_mass(x["q"], x["k"], 1, 1)
    np.testing.assert_allclose(A, _probs_sdpa(x["q"], x["k"]), atol=1e-13)
    np.testing.assert_allclose(A.sum(-1), 1.0, atol=1e-13)


def test_pooled_scores_of_constant_blocks():
    # blocks of identical tokens pool to that token: P = scale * <q, k>
    rng = np.random.default_rng(1)
    qb, kb = rng.standard_normal((3, 4)), rng.standard_normal((2, 4))
    q = np.repeat(qb, 4, axis=0)[None, None]
    k = np.repeat(kb, 5, axis=0)[None, None]
    P = oracle.pooled_scores(q, k, 4, 5)
    np.testing.assert_allclose(P[0, 0], qb @ kb.T / 2.0, atol=1e-14)


@pytest.mark.parametrize("frac,n,k", [(0.25, 8, 2), (0.10, 256, 26), (0.05, 512, 26), (0.03, 16384, 492),
                                      (0.1, 10, 1), (0.3, 10, 3), (0.0001, 8, 1), (1.0, 8, 8), (1.5, 8, 8)])
def test_count_from_fraction(frac, n, k):
    assert oracle.count_from_fraction(frac, n) == k


def _brute_topk(a, k):
    best = None
    for S in itertools.combinations(range(len(a)), k):
        tot = sum(Fraction(float(a[j])) for j in S)
        key = (-tot, S)
        if best is None or key < best:
            best = key
    return list(best[1])


@pytest.mark.parametrize("seed,n,frac,ties", [(0, 8, 0.25, False), (1, 8, 0.5, True), (2, 7, 0.3, True),
                                              (3, 6, 0.5, False), (4, 8, 0.125, True)])
def test_topk_brute_force(seed, n, frac, ties):
    rng = np.random.default_rng(seed)
    A = (rng.integers(0, 4, size=(1, 2, 3, n)).astype(np.float64) if ties else rng.random((1, 2, 3, n)))
    rp, ci = oracle.select_topk(A, frac)
    k = oracle.count_from_fraction(frac, n)
    assert np.all(np.diff(rp) == k) and rp[-1] == A[..., 0].size * k  # kept fraction exactly k/n
    rows = A.reshape(-1, n)
    for r in range(len(rows)):
        got = list(ci[rp[r]:rp[r + 1]])
        assert got == sorted(got)
        assert got == _brute_topk(rows[r], k)
        dropped = np.setdiff1d(np.arange(n), got)
        if len(dropped):
            assert rows[r][got].min() >= rows[r][dropped].max()


def _brute_min_count(a, tau):
    """Smallest number of blocks whose mass reaches tau (exact rationals)."""
    for m in range(1, len(a) + 1):
        if max(sum(Fraction(float(a[j])) for j in S) for S in itertools.combinations(range(len(a)), m)) >= tau:
            return m
    return len(a)


def _dyadic_rows(rng, R, n):
    """Positive rows summing exactly to 1 with dyadic entries (exact float sums)."""
    rows = []
    for _ in range(R):
        w = rng.integers(1, 12, size=n)
        w[rng.integers(0, n)] += 64 - w.sum() if w.sum() < 64 else 0
        rows.append(w / w.sum())
    A = np.array(rows)
    # make the sums exact by using denominators of 64
    A = np.round(A * 64) / 64
    A[:, 0] += 1.0 - A.sum(axis=1)
    assert np.all(A > 0)
    return A


@pytest.mark.parametrize("seed", range(6))
def test_mass_prefix_is_the_shortest_subset(seed):
    rng = np.random.default_rng(seed)
    A = _dyadic_rows(rng, 4, 6).reshape(1, 1, 4, 6)
    for tau in [Fraction(1, 2), Fraction(3, 4), Fraction(29, 64), Fraction(61, 64)]:
        counts = mass_prefix_counts(A, float(tau))
        for r, a in enumerate(A.reshape(-1, 6)):
            assert counts[r] == _brute_min_count(a, tau)


@pytest.mark.parametrize("seed,cap", [(0, 0.5), (1, 0.4), (2, 0.3), (3, 0.9), (4, 0.25), (5, 0.1)])
def test_mass_cap_tau_star_exhaustive(seed, cap):
    rng = np.random.default_rng(seed)
    R, n, mass = 3, 5, 0.95
    A = _dyadic_rows(rng, R, n).reshape(1, 1, R, n)
    rows = A.reshape(-1, n)
    cap_total = Fraction(str(cap)) * R * n

    def D(tau):
        return sum(_brute_min_count(a, tau) for a in rows)

    cand = {Fraction(mass)}
    for a in rows:
        for m in range(1, n + 1):
            for S in itertools.combinations(range(n), m):
                s = sum(Fraction(float(a[j])) for j in S)
                if s <= Fraction(mass):
                    cand.add(s)
    feasible = [t for t in cand if D(t) <= cap_total]
    rp, ci, tau_star = oracle.select_mass_cap(A, mass, cap)
    if feasible:
        assert Fraction(tau_star) == max(feasible)
    else:
        assert np.all(np.diff(rp) == 1)
    counts = np.diff(rp)
    assert counts.sum() <= max(cap_total, R)  # mean density within the cap (or one block per row)
    for r, a in enumerate(rows):
        kept = ci[rp[r]:rp[r + 1]]
        assert list(kept) == sorted(kept)
        kept_by_mass = sorted(kept, key=lambda j: (-a[j], j))
        assert Fraction(float(a[kept].sum())) >= Fraction(tau_star) or counts[r] == n
        if counts[r] > 1:  # minimal: dropping the smallest kept block falls below tau*
            assert Fraction(float(a[kept_by_mass[:-1]].sum())) < Fraction(tau_star)


def test_mass_without_binding_cap_uses_target():
    rng = np.random.default_rng(7)
    A = _dyadic_rows(rng, 4, 6).reshape(1, 1, 4, 6)
    rp, ci, tau = oracle.select_mass_cap(A, 0.75, 1.0)
    assert tau == 0.75
    for r, a in enumerate(A.reshape(-1, 6)):
        assert rp[r + 1] - rp[r] == _brute_min_count(a, Fraction(3, 4))


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (6, 2), (4, 1)])
def test_column_scores_sum_and_reduce_to_probability_column_sums(Hq, Hkv):
    x = {n: v.astype(np.float64) for n, v in tiny_random(30 + Hq, 1, Hq, Hkv, 11, 4).items()}
    _, lse = oracle.dense_attention(x["q"], x["k"], x["v"])
    C = oracle.column_scores(x["q"], x["k"], lse)
    G = Hq // Hkv
    np.testing.assert_allclose(C.sum(-1), G * 11, rtol=1e-13)
    P = _probs_sdpa(x["q"], x["k"])
    for g in range(Hkv):
        np.testing.assert_allclose(C[0, g], P[0, g * G:(g + 1) * G].sum(axis=(0, 1)), rtol=1e-12)


@pytest.mark.parametrize("seed,ties", [(0, False), (1, True), (2, True)])
def test_select_columns_brute_force(seed, ties):
    rng = np.random.default_rng(seed)
    C = rng.integers(0, 3, size=(1, 2, 7)).astype(np.float64) if ties else rng.random((1, 2, 7))
    ci = oracle.select_columns(C, 3)
    for g in range(2):
        assert list(ci[0, g]) == _brute_topk(C[0, g], 3)


# ---- exact block mass -----------------------------------------------------------

@pytest.mark.parametrize("L,bq,bk", [(13, 4, 4), (13, 5, 3), (16, 8, 4), (9, 9, 2)])
def test_exact_block_mass_is_the_block_sum_of_the_probability_matrix(L, bq, bk):
    """Against torch's attention probabilities (SDPA with V = I), summed over
    each block pair and divided by the query block's size (partial blocks
    included); rows sum to 1."""
    x = {n: v.astype(np.float64) for n, v in tiny_random(40 + L + bq, 1, 4, 2, L, 8).items()}
    _, lse = oracle.dense_attention(x["q"], x["k"], x["v"])
    A = oracle.exact_block_mass(x["q"], x["k"], lse, bq, bk)
    P = _probs_sdpa(x["q"], x["k"])
    nqb, nkb = -(-L // bq), -(-L // bk)
    assert A.shape == (1, 4, nqb, nkb)
    for I in range(nqb):
        for J in range(nkb):
            blk = P[0, :, I * bq:(I + 1) * bq, J * bk:(J + 1) * bk]
            np.testing.assert_allclose(A[0, :, I, J], blk.sum(axis=(1, 2)) / blk.shape[1], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(A.sum(-1), 1.0, atol=1e-13)


def test_exact_block_mass_with_one_token_blocks_is_the_probability_matrix():
    x = {n: v.astype(np.float64) for n, v in tiny_random(50, 1, 4, 2, 11, 8).items()}
    _, lse = oracle.dense_attention(x["q"], x["k"], x["v"])
    np.testing.assert_allclose(oracle.exact_block_mass(x["q"], x["k"], lse, 1, 1), _probs_sdpa(x["q"], x["k"]),
                               atol=1e-13)


def test_exact_block_mass_of_one_query_block_is_the_mean_column_mass():
    # one query block over all rows, one-token key blocks, one head per group:
    # A[0, j] = C[j] / L with C the column sums
    x = {n: v.astype(np.float64) for n, v in tiny_random(51, 1, 2, 2, 12, 8).items()}
    _, lse = oracle.dense_attention(x["q"], x["k"], x["v"])
    A = oracle.exact_block_mass(x["q"], x["k"], lse, 12, 1)
    np.testing.assert_allclose(A[0, :, 0], oracle.column_scores(x["q"], x["k"], lse)[0] / 12, rtol=1e-12)


def test_exact_block_mass_of_uniform_attention_is_the_key_share():
    # q = 0: every query attends every key equally, so A[I, J] = |J| / L
    L, bk = 10, 4
    q = np.zeros((1, 2, L, 4))
    k = np.random.default_rng(3).standard_normal((1, 2, L, 4))
    _, lse = oracle.dense_attention(q, k, k)
    A = oracle.exact_block_mass(q, k, lse, 3, bk)
    np.testing.assert_allclose(A, np.broadcast_to(np.array([4, 4, 2]) / L, A.shape), atol=1e-15)
