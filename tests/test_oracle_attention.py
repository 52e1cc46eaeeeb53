"""Pins of the oracle's attention (CPU only).

The oracle is checked against things other than itself:
  * torch's scaled_dot_product_attention in float64 on the CPU (a library
    routine), with boolean masks and grouped kv heads;
  * scipy's logsumexp for the log-sum-exp (a library routine);
  * closed forms: constant V, zero Q, a single allowed key, one-hot V
    (which turns the output into the probability matrix);
  * invariants: an all-ones mask reproduces dense attention, the block-sparse
    and column-sparse gather forms equal dense attention with -inf on the
    masked entries, rows of the probability matrix sum to one, and permuting
    keys together with values changes nothing.
"""

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from workloads import tiny_random

torch.set_default_dtype(torch.float64)


def _sdpa(q, k, v, allowed=None, scale=None):
    """torch reference: [B, H, L, d] float64 arrays, bool mask [B, Hq, L, L]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)) for x in (q, k, v))
    if Hq != Hkv:
        kt = kt.repeat_interleave(Hq // Hkv, dim=1)
        vt = vt.repeat_interleave(Hq // Hkv, dim=1)
    m = None if allowed is None else torch.from_numpy(allowed)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o.numpy()


def _lse_ref(q, k, allowed=None, scale=None):
    Hq, Hkv = q.shape[1], k.shape[1]
    kk = np.repeat(k, Hq // Hkv, axis=1)
    d = q.shape[-1]
    s = (1.0 / np.sqrt(d) if scale is None else scale) * np.einsum("bhid,bhjd->bhij", q, kk)
    b = None if allowed is None else allowed.astype(np.float64)
    return logsumexp(s, axis=-1, b=b)


def _f64(x):
    return {n: oracle.attention.as_f64(a) for n, a in x.items()}


@pytest.mark.parametrize("B,Hq,Hkv,L,d", [(1, 2, 2, 7, 4), (2, 4, 2, 33, 8), (1, 6, 3, 20, 16), (1, 4, 1, 65, 8)])
def test_dense_matches_torch_sdpa_and_logsumexp(B, Hq, Hkv, L, d):
    x = _f64(tiny_random(L + d, B, Hq, Hkv, L, d))
    o, lse = oracle.dense_attention(x["q"], x["k"], x["v"])
    np.testing.assert_allclose(o, _sdpa(x["q"], x["k"], x["v"]), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, _lse_ref(x["q"], x["k"]), rtol=1e-12, atol=1e-12)


def test_dense_row_subset_matches_full():
    x = _f64(tiny_random(3, 1, 2, 2, 40, 8))
    o, lse = oracle.dense_attention(x["q"], x["k"], x["v"])
    rows = np.array([0, 5, 39])
    o2, lse2 = oracle.dense_attention(x["q"], x["k"], x["v"], rows=rows)
    np.testing.assert_array_equal(o2, o[:, :, rows])
    np.testing.assert_array_equal(lse2, lse[:, :, rows])


def test_explicit_scale_is_used():
    x = _f64(tiny_random(4, 1, 2, 2, 9, 4))
    o, lse = oracle.dense_attention(x["q"], x["k"], x["v"], scale=0.3)
    np.testing.assert_allclose(o, _sdpa(x["q"], x["k"], x["v"], scale=0.3), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, _lse_ref(x["q"], x["k"], scale=0.3), rtol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(0)
    B, H, L, d = 1, 3, 17, 5
    q = rng.standard_normal((B, H, L, d))
    k = rng.standard_normal((B, H, L, d))
    # constant V -> O = V
    v = np.broadcast_to(rng.standard_normal(d), (B, H, L, d)).copy()
    o, _ = oracle.dense_attention(q, k, v)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-13)
    # Q = 0 -> uniform weights: O = mean of V, lse = ln L
    v = rng.standard_normal((B, H, L, d))
    o, lse = oracle.dense_attention(np.zeros_like(q), k, v)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=1e-13)
    np.testing.assert_allclose(lse, np.log(L), atol=1e-13)
    # a single allowed key -> o_i = v_j, lse_i = s_ij
    allowed = np.zeros((B, H, L, L), dtype=bool)
    allowed[..., 3] = True
    o, lse = oracle.masked_attention(q, k, v, allowed)
    np.testing.assert_allclose(o, np.broadcast_to(v[:, :, 3:4], o.shape), atol=1e-13)
    s3 = np.einsum("bhid,bhd->bhi", q, k[:, :, 3]) / np.sqrt(d)
    np.testing.assert_allclose(lse, s3, atol=1e-13)


def test_one_hot_v_gives_probability_rows_summing_to_one():
    x = _f64(tiny_random(5, 1, 2, 2, 12, 4))
    L = 12
    v = np.broadcast_to(np.eye(L), (1, 2, L, L)).copy()  # o_i = row i of P
    allowed = np.random.default_rng(1).random((1, 2, L, L)) < 0.5
    allowed[..., 0] = True
    P, _ = oracle.masked_attention(x["q"], x["k"], v, allowed)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-12)
    assert np.all(P[~allowed] == 0.0) and np.all(P[allowed] > 0)
    np.testing.assert_allclose(P, _sdpa(x["q"], x["k"], v, allowed), atol=1e-12)


def test_all_ones_mask_reproduces_dense():
    x = _f64(tiny_random(6, 1, 4, 2, 30, 8))
    allowed = np.ones((1, 4, 30, 30), dtype=bool)
    o1, l1 = oracle.masked_attention(x["q"], x["k"], x["v"], allowed)
    o2, l2 = oracle.dense_attention(x["q"], x["k"], x["v"])
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_masked_matches_torch_with_bool_mask():
    x = _f64(tiny_random(7, 2, 4, 2, 19, 8))
    allowed = np.random.default_rng(2).random((2, 4, 19, 19)) < 0.3
    allowed[..., 5] = True
    o, lse = oracle.masked_attention(x["q"], x["k"], x["v"], allowed)
    np.testing.assert_allclose(o, _sdpa(x["q"], x["k"], x["v"], allowed), atol=1e-12)
    np.testing.assert_allclose(lse, _lse_ref(x["q"], x["k"], allowed), atol=1e-12)


def _random_csr(rng, rows, nkb, max_keep, allow_empty=False):
    kept = []
    for _ in range(rows):
        lo = 0 if allow_empty else 1
        n = rng.integers(lo, max_keep + 1)
        kept.append(np.sort(rng.choice(nkb, size=n, replace=False)))
    rp = np.zeros(rows + 1, dtype=np.int32)
    rp[1:] = np.cumsum([len(r) for r in kept])
    ci = np.concatenate(kept).astype(np.int32) if rp[-1] else np.zeros(0, np.int32)
    return rp, ci


@pytest.mark.parametrize("L,bq,bk", [(32, 8, 8), (37, 8, 4), (30, 16, 8)])
def test_block_sparse_gather_equals_dense_with_minus_inf(L, bq, bk):
    rng = np.random.default_rng(L)
    B, Hq, Hkv, d = 1, 4, 2, 8
    x = _f64(tiny_random(L, B, Hq, Hkv, L, d))
    nqb, nkb = -(-L // bq), -(-L // bk)
    rp, ci = _random_csr(rng, B * Hq * nqb, nkb, nkb, allow_empty=True)
    allowed = oracle.block_token_mask(rp, ci, B, Hq, L, bq, bk)
    o1, l1 = oracle.block_sparse_attention(x["q"], x["k"], x["v"], rp, ci, bq, bk)
    o2, l2 = oracle.masked_attention(x["q"], x["k"], x["v"], allowed)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_array_equal(np.isinf(l1), np.isinf(l2))
    fin = np.isfinite(l2)
    np.testing.assert_allclose(l1[fin], l2[fin], atol=1e-13)
    # rows with an allowed key agree with torch too
    full = allowed.any(-1)
    ref = _sdpa(x["q"], x["k"], x["v"], allowed | ~full[..., None])
    np.testing.assert_allclose(o1[full], ref[full], atol=1e-12)
    # an empty row gives o = 0 and lse = -inf
    assert np.all(o1[~full] == 0) and np.all(np.isneginf(l1[~full]))


def test_block_sparse_full_csr_equals_dense_and_qblock_subset():
    L, bq, bk = 24, 8, 8
    x = _f64(tiny_random(9, 1, 2, 1, L, 4))
    nqb = nkb = 3
    rows = 2 * nqb
    rp = (np.arange(rows + 1) * nkb).astype(np.int32)
    ci = np.tile(np.arange(nkb), rows).astype(np.int32)
    o1, l1 = oracle.block_sparse_attention(x["q"], x["k"], x["v"], rp, ci, bq, bk)
    o2, l2 = oracle.dense_attention(x["q"], x["k"], x["v"])
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
    o3, l3 = oracle.block_sparse_attention(x["q"], x["k"], x["v"], rp, ci, bq, bk, qblocks=[2])
    np.testing.assert_array_equal(o3, o1[:, :, 16:24])


def test_column_sparse_gather_equals_dense_with_minus_inf():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, L, d = 1, 6, 2, 26, 8
    x = _f64(tiny_random(11, B, Hq, Hkv, L, d))
    cols = np.stack([np.sort(rng.choice(L, 7, replace=False)) for _ in range(Hkv)])[None].astype(np.int32)
    o1, l1 = oracle.column_sparse_attention(x["q"], x["k"], x["v"], cols)
    allowed = oracle.column_token_mask(cols, Hq, L)
    o2, l2 = oracle.masked_attention(x["q"], x["k"], x["v"], allowed)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
    np.testing.assert_allclose(o1, _sdpa(x["q"], x["k"], x["v"], allowed), atol=1e-12)


def test_key_permutation_invariance():
    x = _f64(tiny_random(12, 1, 2, 2, 15, 4))
    perm = np.random.default_rng(4).permutation(15)
    o1, l1 = oracle.dense_attention(x["q"], x["k"], x["v"])
    o2, l2 = oracle.dense_attention(x["q"], x["k"][:, :, perm], x["v"][:, :, perm])
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_bf16_decode_is_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x0000], dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.decode_bf16(bits), ref)
