"""GPU parity of the attention forwards against the fp64 oracle.

Small shapes that span several 64-key tiles and query tiles and end in a
ragged tail (L not a multiple of the tile), all element by element.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_bidirectional_attention_amd as sd
from gpu_util import check_out, dev_csr, host_inputs, say, to_dev, to_np
from workloads import score_jump, tiny_random

pytestmark = pytest.mark.gpu


def _inputs(seed, B, Hq, Hkv, L, d, dtype, scale=1.0):
    x = tiny_random(seed, B, Hq, Hkv, L, d, dtype, scale)
    return {n: to_dev(a) for n, a in x.items()}


def _out(q, dtype):
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,Hq,Hkv,L,d", [(1, 4, 2, 300, 128), (2, 2, 2, 200, 64), (1, 3, 1, 64, 128),
                                          (1, 2, 2, 1, 64), (1, 2, 1, 513, 128)])
def test_dense_matches_oracle(dtype, B, Hq, Hkv, L, d):
    say(f"dense {dtype} B={B} Hq={Hq} Hkv={Hkv} L={L} d={d}")
    x = _inputs(L + d, B, Hq, Hkv, L, d, dtype)
    o, lse = _out(x["q"], dtype)
    p = sd.problem_of(x["q"], x["k"])
    sd.sdattn_forward_dense(p, x["q"], x["k"], x["v"], o, lse)
    torch.cuda.synchronize()
    ro, rl = oracle.dense_attention(*(host_inputs(x[n]) for n in "qkv"))
    check_out(to_np(o), ro, to_np(lse), rl, dtype, "dense")


def test_dense_explicit_scale():
    say("dense bf16 softmax_scale=0.03")
    x = _inputs(7, 1, 2, 2, 257, 128, "bf16")
    o, lse = _out(x["q"], "bf16")
    p = sd.problem_of(x["q"], x["k"], softmax_scale=0.03)
    sd.sdattn_forward_dense(p, x["q"], x["k"], x["v"], o, lse)
    torch.cuda.synchronize()
    ro, rl = oracle.dense_attention(*(host_inputs(x[n]) for n in "qkv"), scale=0.03)
    check_out(to_np(o), ro, to_np(lse), rl, "bf16", "dense scale 0.03")


def test_dense_peaked_attention_within_probability_rounding_bound():
    """Logits of +-60: attention concentrates on one key, |o| approaches
    max |v|, and the error is set by two bf16 roundings, of the
    probabilities fed to the PV product and of the stored output, each at
    most 2^-8 relative (plus fp32 noise).  No overflow from the lazy rescale."""
    say("dense bf16 peaked attention (logits ~ +-60)")
    x = _inputs(7, 1, 2, 2, 257, 128, "bf16", scale=1.3)
    o, lse = _out(x["q"], "bf16")
    p = sd.problem_of(x["q"], x["k"], softmax_scale=0.5)
    sd.sdattn_forward_dense(p, x["q"], x["k"], x["v"], o, lse)
    torch.cuda.synchronize()
    hq, hk, hv = (host_inputs(x[n]) for n in "qkv")
    ro, rl = oracle.dense_attention(hq, hk, hv, scale=0.5)
    err = np.abs(to_np(o) - ro)
    vmax = np.abs(oracle.attention.as_f64(hv)).max()
    assert np.isfinite(to_np(o)).all()
    assert err.max() <= 2 * 2.0 ** -8 * vmax + 1e-3
    assert err.mean() <= 2 * 2.0 ** -8 * np.abs(ro).mean() + 1e-4
    assert np.abs(to_np(lse) - rl).max() <= 1e-3


def _random_csr(rng, rows, nkb, kmax, empty_every=0):
    kept, rp = [], [0]
    for r in range(rows):
        n = 0 if (empty_every and r % empty_every == 0) else int(rng.integers(1, kmax + 1))
        kept.append(np.sort(rng.choice(nkb, size=n, replace=False)))
        rp.append(rp[-1] + n)
    ci = np.concatenate(kept).astype(np.int32) if rp[-1] else np.zeros(0, np.int32)
    return np.array(rp, np.int32), ci


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("L,bq,bk,d", [(520, 64, 64, 128), (520, 128, 128, 128), (700, 128, 64, 64),
                                       (700, 64, 128, 128), (384, 128, 128, 64)])
def test_block_sparse_matches_oracle(dtype, L, bq, bk, d):
    say(f"block_sparse {dtype} L={L} bq={bq} bk={bk} d={d}")
    B, Hq, Hkv = 1, 4, 2
    rng = np.random.default_rng(L + bq + bk + d)
    x = _inputs(L * 3 + d, B, Hq, Hkv, L, d, dtype)
    nqb, nkb = -(-L // bq), -(-L // bk)
    rp, ci = _random_csr(rng, B * Hq * nqb, nkb, min(nkb, 4), empty_every=7)
    drp, dci = dev_csr(rp, ci)
    o, lse = _out(x["q"], dtype)
    p = sd.problem_of(x["q"], x["k"])
    sd.sdattn_forward_block_sparse(p, x["q"], x["k"], x["v"], bq, bk, drp, dci, o, lse)
    torch.cuda.synchronize()
    ro, rl = oracle.block_sparse_attention(*(host_inputs(x[n]) for n in "qkv"), rp, ci, bq, bk)
    check_out(to_np(o), ro, to_np(lse), rl, dtype, "block_sparse")


def _per_head_csr(rng, n_pairs, nqb, nkb, counts):
    """CSR whose rows in (batch, head) pair i keep counts[i] blocks each
    (clamped to nkb), a random ascending choice per row."""
    kept, rp = [], [0]
    for i in range(n_pairs):
        for _ in range(nqb):
            n = min(nkb, counts[i])
            kept.append(np.sort(rng.choice(nkb, size=n, replace=False)))
            rp.append(rp[-1] + n)
    ci = np.concatenate(kept).astype(np.int32) if rp[-1] else np.zeros(0, np.int32)
    return np.array(rp, np.int32), ci


@pytest.mark.parametrize("counts_kind", ["uneven", "equal", "one_long"])
@pytest.mark.parametrize("B,Hq,Hkv,L,bq", [(1, 8, 2, 777, 64), (2, 8, 8, 520, 128), (1, 64, 8, 300, 64)])
def test_block_sparse_head_totals_order(counts_kind, B, Hq, Hkv, L, bq):
    """Batch x heads a multiple of eight (up to 64): the block form ranks the
    (batch, head) pairs by their kept-block totals and deals them to the
    XCDs.  Every row is still computed once, by its own workgroup: the output
    equals the oracle element by element whether the totals differ, are all
    equal, or one pair dominates."""
    say(f"block_sparse order {counts_kind} B={B} Hq={Hq} Hkv={Hkv} L={L} bq={bq}")
    d = 128
    rng = np.random.default_rng(B * 1000 + Hq + L + bq)
    x = _inputs(L + Hq, B, Hq, Hkv, L, d, "bf16")
    nqb = nkb = -(-L // bq)
    n_pairs = B * Hq
    if counts_kind == "uneven":
        counts = [int(c) for c in rng.integers(0, nkb + 1, size=n_pairs)]
    elif counts_kind == "equal":
        counts = [max(1, nkb // 3)] * n_pairs
    else:
        counts = [1] * n_pairs
        counts[n_pairs // 2 + 1] = nkb
    rp, ci = _per_head_csr(rng, n_pairs, nqb, nkb, counts)
    drp, dci = dev_csr(rp, ci)
    o, lse = _out(x["q"], "bf16")
    p = sd.problem_of(x["q"], x["k"])
    sd.sdattn_forward_block_sparse(p, x["q"], x["k"], x["v"], bq, bq, drp, dci, o, lse)
    torch.cuda.synchronize()
    ro, rl = oracle.block_sparse_attention(*(host_inputs(x[n]) for n in "qkv"), rp, ci, bq, bq)
    check_out(to_np(o), ro, to_np(lse), rl, "bf16", f"block_sparse order {counts_kind}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Hq,Hkv,L,kcol,d", [(6, 2, 600, 100, 128), (4, 4, 300, 64, 64), (7, 1, 256, 1, 128),
                                             (2, 2, 130, 130, 128), (2, 1, 1500, 1100, 128)])
def test_column_sparse_matches_oracle(dtype, Hq, Hkv, L, kcol, d):
    say(f"column_sparse {dtype} Hq={Hq} Hkv={Hkv} L={L} kcol={kcol} d={d}")
    rng = np.random.default_rng(kcol)
    x = _inputs(kcol + 11, 1, Hq, Hkv, L, d, dtype)
    cols = np.stack([np.sort(rng.choice(L, kcol, replace=False)) for _ in range(Hkv)])[None].astype(np.int32)
    o, lse = _out(x["q"], dtype)
    p = sd.problem_of(x["q"], x["k"])
    sd.sdattn_forward_column_sparse(p, x["q"], x["k"], x["v"], torch.from_numpy(cols).cuda(), kcol, o, lse)
    torch.cuda.synchronize()
    ro, rl = oracle.column_sparse_attention(*(host_inputs(x[n]) for n in "qkv"), cols)
    check_out(to_np(o), ro, to_np(lse), rl, dtype, "column_sparse")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Hq,Hkv,L,kcol,d", [(6, 2, 700, 21, 128), (4, 4, 512, 64, 64), (7, 1, 1000, 130, 128),
                                             (2, 2, 97, 97, 128), (28, 4, 2048, 61, 128), (2, 1, 300, 1, 64),
                                             (3, 1, 1400, 1040, 128), (2, 1, 1100, 1024, 128), (2, 1, 1100, 1025, 128)])
def test_gathered_columns_and_packed_forward(dtype, Hq, Hkv, L, kcol, d):
    """sdattn_gather_columns copies exactly the listed rows; the packed forward
    over them is bit-identical to the column-sparse forward with the same list
    and matches the oracle."""
    say(f"column gather + packed {dtype} Hq={Hq} Hkv={Hkv} L={L} kcol={kcol} d={d}")
    rng = np.random.default_rng(kcol + L)
    x = _inputs(kcol + 23, 1, Hq, Hkv, L, d, dtype)
    cols = np.stack([np.sort(rng.choice(L, kcol, replace=False)) for _ in range(Hkv)])[None].astype(np.int32)
    dcols = torch.from_numpy(cols).cuda()
    p = sd.problem_of(x["q"], x["k"])
    kc = torch.full((1, Hkv, kcol, d), 7, dtype=x["k"].dtype, device="cuda")
    vc = torch.full_like(kc, 7)
    sd.sdattn_gather_columns(p, x["k"], x["v"], dcols, kcol, kc, vc)
    torch.cuda.synchronize()
    hk, hv = host_inputs(x["k"]), host_inputs(x["v"])
    for g in range(Hkv):  # the rows, byte for byte
        np.testing.assert_array_equal(host_inputs(kc)[0, g], hk[0, g, cols[0, g]])
        np.testing.assert_array_equal(host_inputs(vc)[0, g], hv[0, g, cols[0, g]])
    o1, l1 = _out(x["q"], dtype)
    o2, l2 = _out(x["q"], dtype)
    sd.sdattn_forward_column_packed(p, x["q"], kc, vc, kcol, o1, l1)
    sd.sdattn_forward_column_sparse(p, x["q"], x["k"], x["v"], dcols, kcol, o2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16) if dtype == "bf16" else o1, o2.view(torch.int16) if dtype == "bf16" else o2)
    assert torch.equal(l1, l2)
    ro, rl = oracle.column_sparse_attention(host_inputs(x["q"]), hk, hv, cols)
    check_out(to_np(o1), ro, to_np(l1), rl, dtype, "column_packed")


@pytest.mark.parametrize("bq,bk,d", [(64, 64, 128), (128, 128, 128), (128, 64, 128), (128, 128, 64), (128, 64, 64)])
def test_full_csr_equals_dense_and_ones_v(bq, bk, d):
    say(f"full CSR == dense, V=1 -> O=1, bq={bq} bk={bk} d={d}")
    B, Hq, Hkv, L = 1, 2, 2, 640
    x = _inputs(5, B, Hq, Hkv, L, d, "bf16")
    nqb, nkb = -(-L // bq), -(-L // bk)
    rows = B * Hq * nqb
    rp = (np.arange(rows + 1) * nkb).astype(np.int32)
    ci = np.tile(np.arange(nkb), rows).astype(np.int32)
    drp, dci = dev_csr(rp, ci)
    p = sd.problem_of(x["q"], x["k"])
    o1, l1 = _out(x["q"], "bf16")
    o2, l2 = _out(x["q"], "bf16")
    sd.sdattn_forward_block_sparse(p, x["q"], x["k"], x["v"], bq, bk, drp, dci, o1, l1)
    sd.sdattn_forward_dense(p, x["q"], x["k"], x["v"], o2, l2)
    ones = torch.ones_like(x["v"])
    o3, _ = _out(x["q"], "bf16")
    sd.sdattn_forward_block_sparse(p, x["q"], x["k"], ones, bq, bk, drp, dci, o3, None)
    torch.cuda.synchronize()
    if bq == 128 and d == 64:
        assert torch.equal(o1, o2) and torch.equal(l1, l2)  # same 64-key tiles in the same order
    else:  # 32-key tiles (64-query blocks; 128-query blocks at d = 128): same result up to rounding order
        check_out(to_np(o1), to_np(o2), to_np(l1), to_np(l2), "bf16", "full CSR vs dense")
    assert torch.all(o3 == 1.0)


def test_repeat_runs_are_bitwise_identical():
    say("determinism: dense and block-sparse twice")
    x = _inputs(9, 1, 4, 2, 777, 128, "bf16")
    p = sd.problem_of(x["q"], x["k"])
    outs = []
    for _ in range(2):
        o, l = _out(x["q"], "bf16")
        sd.sdattn_forward_dense(p, x["q"], x["k"], x["v"], o, l)
        outs.append((o, l))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_zero_length_is_a_noop():
    p = sd.problem(1, 2, 2, 0, 128, "bf16")
    e = torch.empty(0, device="cuda", dtype=torch.bfloat16)
    sd.sdattn_forward_dense(p, e, e, e, e, None)
    torch.cuda.synchronize()


@pytest.mark.parametrize("jump", [2.0, 4.0])
@pytest.mark.parametrize("form", ["dense", "block128", "block64", "column"])
def test_scores_far_above_the_first_tile(form, jump):
    """The first keys of every row score about 45 (jump 2) or 90 (jump 4)
    nats below the largest later keys, so probabilities taken against the
    first tile's maximum leave the safe range (jump 2) or overflow fp32
    (jump 4); those rows must come out of the checked pass equal to the
    oracle."""
    say(f"score jump {jump} {form}")
    B, Hq, Hkv, L, d = 1, 2, 1, 300, 128
    x = {n: to_dev(a) for n, a in score_jump(int(jump), B, Hq, Hkv, L, d, jump).items()}
    o, lse = _out(x["q"], "bf16")
    p = sd.problem_of(x["q"], x["k"])
    hq, hk, hv = (host_inputs(x[n]) for n in "qkv")
    if form == "dense":
        sd.sdattn_forward_dense(p, x["q"], x["k"], x["v"], o, lse)
        ro, rl = oracle.dense_attention(hq, hk, hv)
    elif form.startswith("block"):
        bq = int(form[5:])
        nqb = -(-L // bq)
        rows = B * Hq * nqb
        rp = (np.arange(rows + 1) * nqb).astype(np.int32)
        ci = np.tile(np.arange(nqb), rows).astype(np.int32)
        drp, dci = dev_csr(rp, ci)
        sd.sdattn_forward_block_sparse(p, x["q"], x["k"], x["v"], bq, bq, drp, dci, o, lse)
        ro, rl = oracle.block_sparse_attention(hq, hk, hv, rp, ci, bq, bq)
    else:
        cols = np.arange(0, L, 2, dtype=np.int32)[None, None]
        sd.sdattn_forward_column_sparse(p, x["q"], x["k"], x["v"], torch.from_numpy(cols).cuda(), cols.shape[-1], o, lse)
        ro, rl = oracle.column_sparse_attention(hq, hk, hv, cols)
    torch.cuda.synchronize()
    assert np.isfinite(to_np(o)).all()
    check_out(to_np(o), ro, to_np(lse), rl, "bf16", f"score jump {jump} {form}")
