"""Dispatch plan of the block-sparse forward (sdattn_block_plan).

The plan is a scheduling choice, not part of what the method computes, so
it is checked by what it must satisfy: it equals the rule written out on the
host below (segments of consecutive query blocks ranked by their kept
blocks, ties in the plain order, dealt to the eight XCDs in snake order, the
rows of a segment longest first), it
is a permutation of the block rows, it evens the XCDs' kept blocks under
head-skewed budgets (Step-dLLM, Abstract: head-adaptive budget), and the
planned forward is bit-identical to the unplanned one (each row is computed
by one workgroup either way) and within tolerance of the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_bidirectional_attention_amd as sd
from gpu_util import check_out, dev_csr, host_inputs, say, to_dev, to_np
from workloads import tiny_random

pytestmark = pytest.mark.gpu


def _segment_rows(block_q, nqt):
    """Rows one XCD runs at once: 32 CUs times the forward's workgroups per
    CU (four 64-query or three 128-query blocks), lowered to the largest
    divisor of nqt."""
    in_flight = 32 * (4 if block_q == 64 else 3)
    if nqt <= in_flight:
        return nqt
    s = in_flight
    while s > 1 and nqt % s:
        s -= 1
    return s


def _snake(s):
    j, x = divmod(s, 8)
    return 8 * j + (7 - x if j % 2 else x)


def host_plan(row_ptr, rows, nqt, block_q):
    seg = _segment_rows(block_q, nqt)
    n_seg = rows // seg
    if nqt % seg or n_seg % 8 or n_seg > (1 << 20) or seg > 1024:
        return np.arange(rows)
    parts = nqt // seg

    def first_row(s):
        return (s // parts) * nqt + (s % parts) * seg

    tot = [int(row_ptr[first_row(s) + seg]) - int(row_ptr[first_row(s)]) for s in range(n_seg)]
    ranked = sorted(range(n_seg), key=lambda s: (-tot[s], _snake(s)))
    ne = np.diff(np.asarray(row_ptr, np.int64))
    # within a segment: most kept blocks first, ties in row order
    inner = {s: sorted(range(seg), key=lambda t: (-ne[first_row(s) + t], t)) for s in range(n_seg)}
    plan = np.empty(rows, np.int64)
    for i in range(rows):
        x, m = i % 8, i // 8
        k, j = divmod(m, seg)
        r = 8 * k + (7 - x if k % 2 else x)
        plan[i] = first_row(ranked[r]) + inner[ranked[r]][j]
    return plan


def _skewed_csr(rng, pairs, nqb, nkb, per_pair):
    """Rows of pair i keep per_pair[i] blocks (clamped to nkb), a random ascending choice each."""
    kept, rp = [], [0]
    for i in range(pairs):
        k = int(min(max(per_pair[i], 0), nkb))
        for _ in range(nqb):
            kept.append(np.sort(rng.choice(nkb, size=k, replace=False)))
            rp.append(rp[-1] + k)
    ci = np.concatenate(kept).astype(np.int32) if rp[-1] else np.zeros(0, np.int32)
    return np.array(rp, np.int32), ci


def _gpu_plan(p, bq, bk, drp, rows):
    plan = torch.full((max(rows, 1),), -7, dtype=torch.int32, device="cuda")
    sd.sdattn_block_plan(p, bq, bk, drp, plan)
    torch.cuda.synchronize()
    return plan, plan.cpu().numpy()[:rows].astype(np.int64)


@pytest.mark.parametrize("B,Hq,L,bq,skew", [
    (1, 32, 8192, 64, False),     # 64-query blocks, whole heads per segment
    (1, 32, 8192, 64, True),
    (1, 32, 65536, 128, False),   # 128-query blocks, eight segments per head
    (1, 32, 65536, 128, True),
    (2, 8, 16384, 128, True),     # two batches
    (1, 4, 520, 64, False),       # segments do not fill rounds of eight: identity
    (1, 3, 700, 128, True),
])
def test_plan_is_the_ranked_snake_deal(B, Hq, L, bq, skew):
    say(f"plan B={B} Hq={Hq} L={L} bq={bq} skew={skew}")
    rng = np.random.default_rng(L + Hq + bq)
    nqt = -(-L // bq)
    nkb = -(-L // bq)
    pairs = B * Hq
    if skew:
        per_pair = np.round(np.exp(rng.uniform(np.log(1), np.log(min(nkb, 64)), pairs))).astype(int)
    else:
        per_pair = np.full(pairs, max(1, nkb // 20))
    rp, ci = _skewed_csr(rng, pairs, nqt, nkb, per_pair)
    rows = pairs * nqt
    p = sd.problem(B, Hq, Hq, L, 128, "bf16")
    drp, _ = dev_csr(rp, ci)
    _, plan = _gpu_plan(p, bq, bq, drp, rows)
    assert np.array_equal(np.sort(plan), np.arange(rows))
    assert np.array_equal(plan, host_plan(rp, rows, nqt, bq))
    if not skew and _segment_rows(bq, nqt) * 8 <= rows and rows % (8 * _segment_rows(bq, nqt)) == 0:
        # equal totals: segment s on XCD s mod 8 in round s / 8
        seg = _segment_rows(bq, nqt)
        ids = np.arange(rows)
        seg_of_row = plan // seg
        assert np.array_equal(seg_of_row % 8, ids % 8)


def test_plan_evens_the_xcds_under_a_head_skewed_budget():
    """One head keeps 16 times the blocks of the others (64K shape, 128-query
    blocks): the plan's XCD totals are within 2% of each other, where whole
    heads per XCD would leave one XCD with over twice the mean."""
    say("plan XCD balance, one heavy head")
    rng = np.random.default_rng(11)
    B, Hq, L, bq = 1, 32, 65536, 128
    nqt = nkb = L // bq
    per_pair = np.full(B * Hq, 8)
    per_pair[5] = 128
    rp, ci = _skewed_csr(rng, B * Hq, nqt, nkb, per_pair)
    rows = B * Hq * nqt
    p = sd.problem(B, Hq, Hq, L, 128, "bf16")
    drp, _ = dev_csr(rp, ci)
    _, plan = _gpu_plan(p, bq, bq, drp, rows)
    ne = np.diff(rp)[plan]
    xcd = np.array([ne[x::8].sum() for x in range(8)])
    assert xcd.max() <= 1.02 * xcd.mean()
    whole = np.array([sum(per_pair[h] * nqt for h in range(x, B * Hq, 8)) for x in range(8)])
    assert whole.max() > 2 * whole.mean()


@pytest.mark.parametrize("L,bq,bk,d,dtype", [(1000, 64, 64, 128, "bf16"), (777, 128, 128, 128, "bf16"),
                                             (1300, 128, 64, 64, "bf16"), (520, 64, 128, 128, "bf16"),
                                             (700, 128, 128, 64, "f32")])
def test_planned_forward_is_the_unplanned_one(L, bq, bk, d, dtype):
    say(f"planned forward {dtype} L={L} bq={bq} bk={bk} d={d}")
    B, Hq, Hkv = 1, 16, 4
    rng = np.random.default_rng(L * 3 + bq + bk)
    x = {n: to_dev(a) for n, a in tiny_random(L + d, B, Hq, Hkv, L, d, dtype).items()}
    nqt, nkb = -(-L // bq), -(-L // bk)
    per_pair = rng.integers(0, nkb + 1, B * Hq)
    per_pair[0] = nkb  # a full row pattern in one head, empty rows where the count is 0
    rp, ci = _skewed_csr(rng, B * Hq, nqt, nkb, per_pair)
    drp, dci = dev_csr(rp, ci)
    p = sd.problem_of(x["q"], x["k"])
    plan, plan_h = _gpu_plan(p, bq, bk, drp, B * Hq * nqt)
    assert np.array_equal(np.sort(plan_h), np.arange(B * Hq * nqt))
    o1, l1 = torch.empty_like(x["q"]), torch.empty(x["q"].shape[:3], dtype=torch.float32, device="cuda")
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    sd.sdattn_forward_block_sparse(p, x["q"], x["k"], x["v"], bq, bk, drp, dci, o1, l1)
    sd.sdattn_forward_block_sparse_planned(p, x["q"], x["k"], x["v"], bq, bk, drp, dci, plan, o2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ro, rl = oracle.block_sparse_attention(*(host_inputs(x[n]) for n in "qkv"), rp, ci, bq, bk)
    check_out(to_np(o2), ro, to_np(l2), rl, dtype, "planned block_sparse")


def test_planned_forward_writes_nothing_for_entries_outside_the_rows():
    """A plan entry that names no block row leaves that workgroup idle: the
    rows the plan does name are computed, the others keep what they held."""
    say("planned forward, plan with out-of-range entries")
    B, Hq, Hkv, L, d, bq = 1, 4, 4, 256, 128, 64
    x = {n: to_dev(a) for n, a in tiny_random(3, B, Hq, Hkv, L, d, "bf16").items()}
    nqt = L // bq
    rows = B * Hq * nqt
    rp = np.arange(rows + 1, dtype=np.int32) * 2
    ci = np.tile(np.array([0, 2], np.int32), rows)
    drp, dci = dev_csr(rp, ci)
    p = sd.problem_of(x["q"], x["k"])
    plan = torch.arange(rows, dtype=torch.int32, device="cuda")
    plan[3] = rows + 5
    plan[7] = -1
    o = torch.full_like(x["q"], 7.0)
    lse = torch.full(x["q"].shape[:3], 7.0, dtype=torch.float32, device="cuda")
    sd.sdattn_forward_block_sparse_planned(p, x["q"], x["k"], x["v"], bq, bq, drp, dci, plan, o, lse)
    ref, rl = torch.empty_like(o), torch.empty_like(lse)
    sd.sdattn_forward_block_sparse(p, x["q"], x["k"], x["v"], bq, bq, drp, dci, ref, rl)
    torch.cuda.synchronize()
    skipped = np.zeros(rows, bool)
    skipped[[3, 7]] = True
    o_rows = o.view(B * Hq, nqt, bq, d)
    ref_rows = ref.view(B * Hq, nqt, bq, d)
    for r in range(rows):
        bh, qt = divmod(r, nqt)
        if skipped[r]:
            assert bool((o_rows[bh, qt] == 7.0).all())
        else:
            assert torch.equal(o_rows[bh, qt], ref_rows[bh, qt])
