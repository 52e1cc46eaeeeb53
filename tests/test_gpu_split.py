"""Split rows of the block-sparse forward (sdattn_block_split_plan,
sdattn_forward_block_sparse_split).

Cutting a long block row into chunks of its kept blocks and combining the
chunks' partial results by their log-sum-exps (the online-softmax merge of
partial rows, LoSA section 3) computes the same attention as the whole row.
So the split forward is checked against the oracle element by element, and
against the unsplit forward: rows that are not cut are bit-identical to it.
The split plan is a scheduling choice and is checked against its rule written
out on the host: which rows are cut and into how many chunks, that every
(row, chunk) is dealt to exactly one workgroup, where the chunks' partial
slots lie, and that the plan's other entries are the dispatch plan's.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_bidirectional_attention_amd as sd
from gpu_util import check_out, dev_csr, host_inputs, say, to_dev, to_np
from workloads import tiny_random

pytestmark = pytest.mark.gpu

ROW_MASK = (1 << 24) - 1


def _slots(block_q):
    # workgroups the GPU holds at once: 256 CUs times four 64-query or three 128-query blocks
    return 256 * (4 if block_q == 64 else 3)


def host_split(rp, rows, block_q):
    """Chunk length T and chunk count per row, as the split plan defines them."""
    slots = _slots(block_q)
    rp = np.asarray(rp, np.int64)
    nnz = int(rp[rows] - rp[0])
    T = max(4, -(-nnz // slots))
    ne = np.diff(rp[:rows + 1])
    c = np.where(ne > T, np.minimum(8, -(-ne // T)), 1)
    return T, c.astype(np.int64)


def _skewed_csr(rng, pairs, nqb, nkb, per_pair, empty_rows=()):
    kept, rp = [], [0]
    for i in range(pairs):
        k = int(min(max(per_pair[i], 0), nkb))
        for j in range(nqb):
            kk = 0 if (i * nqb + j) in empty_rows else k
            kept.append(np.sort(rng.choice(nkb, size=kk, replace=False)))
            rp.append(rp[-1] + kk)
    ci = np.concatenate(kept).astype(np.int32) if rp[-1] else np.zeros(0, np.int32)
    return np.array(rp, np.int32), ci


def _split_plan(p, bq, bk, drp):
    wsb = sd.sdattn_block_split_workspace(p, bq, bk)
    ws = torch.full((max(wsb, 4),), 0x5A, dtype=torch.uint8, device="cuda")
    sd.sdattn_block_split_plan(p, bq, bk, drp, ws, wsb)
    torch.cuda.synchronize()
    return ws, wsb


def _read_plan(ws, rows, block_q):
    slots = _slots(block_q)
    n_items = rows + 2 * slots
    w = ws.view(torch.int32).cpu().numpy().astype(np.int64)
    items = w[:n_items]
    slot_base = w[n_items:n_items + rows]
    counts = w[n_items + rows:n_items + rows + 2]
    off = n_items + rows + 2
    split_rows = w[off:off + slots]
    plan = w[off + slots:off + slots + rows]
    return items, slot_base, counts, split_rows, plan


def check_split_plan(ws, rp, rows, nqt, block_q, p, block_k, drp):
    T, c = host_split(rp, rows, block_q)
    items, slot_base, counts, split_rows, plan = _read_plan(ws, rows, block_q)
    split = np.nonzero(c > 1)[0]
    assert counts[0] == len(split) and counts[1] == T
    # the dispatch plan the items are built from is sdattn_block_plan's
    ref_plan = torch.empty(rows, dtype=torch.int32, device="cuda")
    sd.sdattn_block_plan(p, block_q, block_k, drp, ref_plan)
    torch.cuda.synchronize()
    assert np.array_equal(plan, ref_plan.cpu().numpy())
    # every chunk of the split rows first (row order, chunks in order: chunk k
    # of row r at its partial slot), then idle up to a multiple of 8
    chunk_items = [(r | ((c[r] - 1) << 27)) | (k << 24) for r in split for k in range(c[r])]
    CS = len(chunk_items)
    C8 = (CS + 7) // 8 * 8
    assert CS < 2 * _slots(block_q)
    assert np.array_equal(items[:CS], np.array(chunk_items, np.int64))
    assert np.all(items[CS:C8] == -1)
    # then the dispatch plan with the split rows idle, then idle
    assert np.array_equal(items[C8:C8 + rows], np.where(c[plan] > 1, -1, plan))
    assert np.all(items[C8 + rows:] == -1)
    # every (row, chunk) exactly once
    live = items[items >= 0]
    pairs = sorted(zip((live & ROW_MASK).tolist(), ((live >> 24) & 7).tolist()))
    assert pairs == sorted((r, k) for r in range(rows) for k in range(c[r]))
    # split-row list and partial slots: consecutive ranges in row order
    assert np.array_equal(split_rows[:len(split)], split | ((c[split] - 1) << 27))
    starts = np.concatenate([[0], np.cumsum(c[split])[:-1]]) if len(split) else np.zeros(0, np.int64)
    assert np.array_equal(slot_base[split], starts)
    assert np.all(slot_base[c == 1] == -1)
    return T, c


@pytest.mark.parametrize("B,L,bq,bk,d", [(1, 1000, 64, 64, 128), (1, 777, 128, 128, 128), (1, 1300, 128, 64, 64),
                                         (1, 520, 64, 128, 128), (1, 2048, 64, 64, 64), (2, 600, 64, 64, 128),
                                         (2, 900, 128, 128, 64)])
def test_split_forward_matches_the_oracle(B, L, bq, bk, d):
    """One head keeps every key block, the others a few, some rows none: long
    rows are cut (chunk length 4 blocks at these sizes), and the merged rows
    match the oracle; rows that are not cut equal the unsplit forward bit for
    bit."""
    say(f"split forward B={B} L={L} bq={bq} bk={bk} d={d}")
    Hq, Hkv = 8 // B, 2
    rng = np.random.default_rng(L + 7 * bq + bk + d)
    x = {n: to_dev(a) for n, a in tiny_random(L + d + 1, B, Hq, Hkv, L, d, "bf16").items()}
    nqt, nkb = -(-L // bq), -(-L // bk)
    per_pair = rng.integers(1, 4, B * Hq)
    per_pair[3] = nkb
    per_pair[6] = max(1, nkb // 2)
    rp, ci = _skewed_csr(rng, B * Hq, nqt, nkb, per_pair, empty_rows={1, 3 * nqt + 1})
    rows = B * Hq * nqt
    drp, dci = dev_csr(rp, ci)
    p = sd.problem_of(x["q"], x["k"])
    ws, wsb = _split_plan(p, bq, bk, drp)
    T, c = check_split_plan(ws, rp, rows, nqt, bq, p, bk, drp)
    assert (c > 1).sum() > 0, "the pattern should have rows to cut"
    o = torch.full_like(x["q"], 3.0)
    lse = torch.full(x["q"].shape[:3], 3.0, dtype=torch.float32, device="cuda")
    sd.sdattn_forward_block_sparse_split(p, x["q"], x["k"], x["v"], bq, bk, drp, dci, ws, o, lse, ws_bytes=wsb)
    o1, l1 = torch.empty_like(o), torch.empty_like(lse)
    sd.sdattn_forward_block_sparse(p, x["q"], x["k"], x["v"], bq, bk, drp, dci, o1, l1)
    torch.cuda.synchronize()
    ro, rl = oracle.block_sparse_attention(*(host_inputs(x[n]) for n in "qkv"), rp, ci, bq, bk)
    check_out(to_np(o), ro, to_np(lse), rl, "bf16", "split block_sparse")
    qa = o.view(B * Hq, L, d)
    qb = o1.view(B * Hq, L, d)
    for bh in range(B * Hq):
        for qt in range(nqt):
            r = bh * nqt + qt
            sl = slice(qt * bq, min(L, (qt + 1) * bq))
            if c[r] == 1:
                assert torch.equal(qa[bh, sl], qb[bh, sl]), f"row {r} (not cut) differs from the unsplit forward"
                assert torch.equal(lse.view(B * Hq, L)[bh, sl], l1.view(B * Hq, L)[bh, sl])


def test_split_forward_is_repeatable_and_f32_computes_whole_rows():
    """The workspace holds the partial results; a second call over the same
    plan gives the same bytes.  float32 problems compute every row whole
    (bit-identical to the unsplit float32 forward)."""
    say("split forward twice; f32 split forward")
    B, Hq, Hkv, L, d, bq = 1, 4, 4, 640, 128, 64
    rng = np.random.default_rng(17)
    nqt = nkb = L // bq
    rp, ci = _skewed_csr(rng, B * Hq, nqt, nkb, [nkb, 2, 9, 3])
    drp, dci = dev_csr(rp, ci)
    for dtype in ("bf16", "f32"):
        x = {n: to_dev(a) for n, a in tiny_random(5, B, Hq, Hkv, L, d, dtype).items()}
        p = sd.problem_of(x["q"], x["k"])
        ws, wsb = _split_plan(p, bq, bq, drp)
        outs = []
        for _ in range(2):
            o = torch.empty_like(x["q"])
            lse = torch.empty(x["q"].shape[:3], dtype=torch.float32, device="cuda")
            sd.sdattn_forward_block_sparse_split(p, x["q"], x["k"], x["v"], bq, bq, drp, dci, ws, o, lse)
            outs.append((o, lse))
        torch.cuda.synchronize()
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
        ro, rl = oracle.block_sparse_attention(*(host_inputs(x[n]) for n in "qkv"), rp, ci, bq, bq)
        check_out(to_np(outs[0][0]), ro, to_np(outs[0][1]), rl, dtype, f"split {dtype}")
        if dtype == "f32":
            o1, l1 = torch.empty_like(x["q"]), torch.empty_like(outs[0][1])
            sd.sdattn_forward_block_sparse(p, x["q"], x["k"], x["v"], bq, bq, drp, dci, o1, l1)
            torch.cuda.synchronize()
            assert torch.equal(o1, outs[0][0]) and torch.equal(l1, outs[0][1])


def test_even_rows_are_not_cut_and_match_the_planned_forward():
    """A top-k pattern at the 8K LLaDA shape (every row 13 kept blocks, far
    below one slot's share): nothing is cut, and the split forward is the
    planned forward bit for bit."""
    say("split plan of an even 8K pattern")
    B, Hq, L, d, bq = 1, 32, 8192, 128, 64
    nqt = nkb = L // bq
    rng = np.random.default_rng(23)
    rp, ci = _skewed_csr(rng, B * Hq, nqt, nkb, np.full(B * Hq, 13))
    x = {n: to_dev(a) for n, a in tiny_random(29, B, Hq, Hq, L, d, "bf16").items()}
    p = sd.problem_of(x["q"], x["k"])
    drp, dci = dev_csr(rp, ci)
    ws, wsb = _split_plan(p, bq, bq, drp)
    T, c = check_split_plan(ws, rp, B * Hq * nqt, nqt, bq, p, bq, drp)
    assert (c > 1).sum() == 0
    o = torch.empty_like(x["q"])
    lse = torch.empty(x["q"].shape[:3], dtype=torch.float32, device="cuda")
    sd.sdattn_forward_block_sparse_split(p, x["q"], x["k"], x["v"], bq, bq, drp, dci, ws, o, lse)
    plan = torch.empty(B * Hq * nqt, dtype=torch.int32, device="cuda")
    sd.sdattn_block_plan(p, bq, bq, drp, plan)
    o1, l1 = torch.empty_like(o), torch.empty_like(lse)
    sd.sdattn_forward_block_sparse_planned(p, x["q"], x["k"], x["v"], bq, bq, drp, dci, plan, o1, l1)
    torch.cuda.synchronize()
    assert torch.equal(o, o1) and torch.equal(lse, l1)


def test_split_at_the_8k_shape_with_one_dense_head():
    """The case the split exists for: at the 8K LLaDA shape one head keeps
    every key block (128 per row) and the others 4.  The dense head's rows
    are cut into chunks of T blocks; sampled query blocks of every head match
    the oracle, and the whole output matches the unsplit forward within the
    bf16 tolerance."""
    say("split forward, 8K, one dense head")
    B, Hq, L, d, bq = 1, 32, 8192, 128, 64
    nqt = nkb = L // bq
    rng = np.random.default_rng(31)
    per_pair = np.full(B * Hq, 4)
    per_pair[7] = nkb
    rp, ci = _skewed_csr(rng, B * Hq, nqt, nkb, per_pair)
    rows = B * Hq * nqt
    x = {n: to_dev(a) for n, a in tiny_random(37, B, Hq, Hq, L, d, "bf16").items()}
    p = sd.problem_of(x["q"], x["k"])
    drp, dci = dev_csr(rp, ci)
    ws, wsb = _split_plan(p, bq, bq, drp)
    T, c = check_split_plan(ws, rp, rows, nqt, bq, p, bq, drp)
    assert T == 32 and np.all(c[7 * nqt:8 * nqt] == 4) and (c > 1).sum() == nqt
    o = torch.empty_like(x["q"])
    lse = torch.empty(x["q"].shape[:3], dtype=torch.float32, device="cuda")
    sd.sdattn_forward_block_sparse_split(p, x["q"], x["k"], x["v"], bq, bq, drp, dci, ws, o, lse)
    o1, l1 = torch.empty_like(o), torch.empty_like(lse)
    sd.sdattn_forward_block_sparse(p, x["q"], x["k"], x["v"], bq, bq, drp, dci, o1, l1)
    torch.cuda.synchronize()
    check_out(to_np(o), to_np(o1), to_np(lse), to_np(l1), "bf16", "split vs unsplit, 8K")
    qblocks = [0, 5, 64, 127]
    xs = {n: host_inputs(x[n]) for n in "qkv"}
    for h in (0, 7, 31):
        sub = {n: xs[n][:, h:h + 1] for n in "qkv"}
        r0 = h * nqt
        rph = rp[r0:r0 + nqt + 1] - rp[r0]
        cih = ci[rp[r0]:rp[r0 + nqt]]
        ro, rl = oracle.block_sparse_attention(sub["q"], sub["k"], sub["v"], rph, cih, bq, bq, qblocks=qblocks)
        got = np.concatenate([to_np(o[0, h, qb * bq:(qb + 1) * bq]) for qb in qblocks])
        gl = np.concatenate([to_np(lse[0, h, qb * bq:(qb + 1) * bq]) for qb in qblocks])
        check_out(got, np.asarray(ro).reshape(got.shape), gl, np.asarray(rl).reshape(gl.shape), "bf16",
                  f"split 8K head {h}")
