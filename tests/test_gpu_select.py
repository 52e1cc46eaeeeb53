"""GPU parity of the pattern selectors against the fp64 oracle.

Index sets must match the oracle exactly except for candidates whose
oracle score lies within 1e-5 (relative) of the row's cut; debug scores
(pooled mass, column scores) within 1e-5 relative.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_bidirectional_attention_amd as sd
from gpu_util import CUT_REL, SCORE_REL, check_topk_rows, csr_rows, host_inputs, say, to_dev
from workloads import WORKLOADS, make_step, tiny_random
from workloads.configs import scaled

pytestmark = pytest.mark.gpu


def _dev(x):
    return {n: to_dev(a) for n, a in x.items()}


def _select_blocks(x, bq, bk, budget):
    p = sd.problem_of(x["q"], x["k"])
    ws_bytes, nnz = sd.sdattn_select_blocks_workspace(p, bq, bk, budget)
    L = x["q"].shape[2]
    rows = x["q"].shape[0] * x["q"].shape[1] * (-(-L // bq))
    nkb = -(-L // bk)
    rp = torch.empty(rows + 1, dtype=torch.int32, device="cuda")
    ci = torch.full((max(nnz, 1),), -1, dtype=torch.int32, device="cuda")
    mass = torch.empty(rows * nkb, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    sd.sdattn_select_blocks(p, x["q"], x["k"], bq, bk, budget, rp, ci, nnz, mass, ws, ws_bytes)
    torch.cuda.synchronize()
    return rp.cpu().numpy(), ci.cpu().numpy(), mass.cpu().numpy().astype(np.float64).reshape(rows, nkb)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Hq,Hkv,L,bq,bk,frac", [(4, 2, 1000, 64, 64, 0.25), (4, 4, 1300, 128, 128, 0.1),
                                                 (2, 1, 700, 128, 64, 0.3), (3, 3, 4096, 64, 64, 0.05),
                                                 (2, 2, 65, 64, 64, 0.5)])
def test_topk_selection_matches_oracle(dtype, Hq, Hkv, L, bq, bk, frac):
    say(f"select_blocks topk {dtype} Hq={Hq} Hkv={Hkv} L={L} bq={bq} bk={bk} frac={frac}")
    x = _dev(tiny_random(L + Hq, 1, Hq, Hkv, L, 128, dtype, scale=1.0))
    rp, ci, mass = _select_blocks(x, bq, bk, sd.topk_budget(frac))
    hq, hk = host_inputs(x["q"]), host_inputs(x["k"])
    A = oracle.pooled_mass(hq, hk, bq, bk)
    nkb = A.shape[-1]
    A = A.reshape(-1, nkb)
    np.testing.assert_allclose(mass, A, rtol=SCORE_REL, atol=1e-30)
    k = oracle.count_from_fraction(frac, nkb)
    assert rp[0] == 0 and np.all(np.diff(rp) == k)
    n_ex = check_topk_rows(csr_rows(rp, ci), A, k, "topk")
    say(f"  rows with exempt near-cut differences: {n_ex} of {len(A)}")


def test_topk_on_planted_workload_shape():
    w = scaled(WORKLOADS["sparsed_32k"], seq_len=4096, q_heads=8, kv_heads=8)
    say(f"select_blocks topk planted {w.name} L={w.seq_len}")
    x = _dev(make_step(w, w.select_step))
    rp, ci, mass = _select_blocks(x, w.block, w.block, sd.topk_budget(w.keep_frac))
    A = oracle.pooled_mass(host_inputs(x["q"]), host_inputs(x["k"]), w.block, w.block).reshape(-1, w.n_blocks)
    check_topk_rows(csr_rows(rp, ci), A, oracle.count_from_fraction(w.keep_frac, w.n_blocks), "topk planted")


def _check_mass_rows(rp, ci, A, tau_ref, mass, cap):
    """Row counts within [n(tau*(1-e)), n(tau*(1+e))] of the oracle's cumulative
    arrays; each row is that prefix of the (A desc, J asc) order up to exempt
    near-cut swaps; the total respects the cap."""
    R, n = A.shape
    counts = np.diff(rp)
    allowed = max(R, int(np.floor(cap * R * n + 1e-9)))
    assert counts.sum() <= allowed
    for r in range(R):
        a = A[r]
        order = np.lexsort((np.arange(n), -a))
        c = np.cumsum(a[order])
        lo = max(1, int(np.searchsorted(c, tau_ref * (1 - CUT_REL), side="left")) + 1)
        hi = max(1, int(np.searchsorted(c, tau_ref * (1 + CUT_REL), side="left")) + 1)
        cnt = counts[r]
        assert min(lo, n) <= cnt <= min(hi, n), f"row {r}: count {cnt} outside [{lo}, {hi}]"
        g = np.sort(ci[rp[r]:rp[r + 1]])
        ref = np.sort(order[:cnt])
        if not np.array_equal(g, ref):
            cut = a[order[cnt - 1]]
            assert np.all(a[np.setdiff1d(g, ref)] >= cut * (1 - CUT_REL))
            assert np.all(a[np.setdiff1d(ref, g)] <= cut * (1 + CUT_REL))


@pytest.mark.parametrize("mass,cap,L,bq", [(0.95, 0.10, 4096, 64), (0.95, 1.0, 2000, 64), (0.5, 0.3, 3000, 128),
                                           (0.95, 0.02, 2048, 64)])
def test_mass_cap_selection_matches_oracle(mass, cap, L, bq):
    w = scaled(WORKLOADS["llada8b_8k"], seq_len=L, q_heads=8, kv_heads=8, block=bq)
    say(f"select_blocks mass={mass} cap={cap} L={L} bq={bq}")
    x = _dev(make_step(w, 0))
    rp, ci, gmass = _select_blocks(x, bq, bq, sd.mass_budget(mass, cap))
    A4 = oracle.pooled_mass(host_inputs(x["q"]), host_inputs(x["k"]), bq, bq)
    A = A4.reshape(-1, A4.shape[-1])
    np.testing.assert_allclose(gmass, A, rtol=SCORE_REL, atol=1e-30)
    rrp, rci, tau = oracle.select_mass_cap(A4, mass, cap)
    say(f"  oracle tau*={tau:.6f} nnz={rrp[-1]} gpu nnz={rp[-1]} density={rp[-1] / A.size:.4f}")
    _check_mass_rows(rp, ci, A, tau, mass, cap)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Hq,Hkv,L,kcol,d", [(6, 2, 700, 21, 128), (4, 4, 512, 64, 64), (7, 1, 1000, 30, 128),
                                             (2, 2, 97, 97, 128)])
def test_column_selection_matches_oracle(dtype, Hq, Hkv, L, kcol, d):
    say(f"select_columns {dtype} Hq={Hq} Hkv={Hkv} L={L} kcol={kcol} d={d}")
    x = _dev(tiny_random(kcol + L, 1, Hq, Hkv, L, d, dtype))
    p = sd.problem_of(x["q"], x["k"])
    o = torch.empty_like(x["q"])
    lse = torch.empty(x["q"].shape[:3], dtype=torch.float32, device="cuda")
    sd.sdattn_forward_dense(p, x["q"], x["k"], x["v"], o, lse)
    ws_bytes = sd.sdattn_select_columns_workspace(p, kcol)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    cols = torch.full((1, Hkv, kcol), -1, dtype=torch.int32, device="cuda")
    C = torch.empty((1, Hkv, L), dtype=torch.float64, device="cuda")
    sd.sdattn_select_columns(p, x["q"], x["k"], lse, kcol, cols, C, ws, ws_bytes)
    torch.cuda.synchronize()
    hq, hk = host_inputs(x["q"]), host_inputs(x["k"])
    _, rl = oracle.dense_attention(hq, hk, host_inputs(x["v"]))
    Cref = oracle.column_scores(hq, hk, rl)
    np.testing.assert_allclose(C.cpu().numpy(), Cref, rtol=SCORE_REL)
    np.testing.assert_allclose(C.cpu().numpy().sum(-1), Hq // Hkv * L, rtol=1e-5)
    check_topk_rows(cols.cpu().numpy()[0], Cref[0], kcol, "columns")


def test_planted_columns_are_found():
    w = scaled(WORKLOADS["pulsecol_dream7b_16k"], seq_len=2048, q_heads=14, kv_heads=2, n_stripe_columns=40)
    say("select_columns on planted stripes")
    x = _dev(make_step(w, 0))
    p = sd.problem_of(x["q"], x["k"])
    o = torch.empty_like(x["q"])
    lse = torch.empty(x["q"].shape[:3], dtype=torch.float32, device="cuda")
    sd.sdattn_forward_dense(p, x["q"], x["k"], x["v"], o, lse)
    kcol = oracle.count_from_fraction(w.column_keep_frac, w.seq_len)
    ws_bytes = sd.sdattn_select_columns_workspace(p, kcol)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    cols = torch.empty((1, 2, kcol), dtype=torch.int32, device="cuda")
    sd.sdattn_select_columns(p, x["q"], x["k"], lse, kcol, cols, None, ws, ws_bytes)
    torch.cuda.synchronize()
    hq, hk = host_inputs(x["q"]), host_inputs(x["k"])
    _, rl = oracle.dense_attention(hq, hk, host_inputs(x["v"]))
    Cref = oracle.column_scores(hq, hk, rl)
    check_topk_rows(cols.cpu().numpy()[0], Cref[0], kcol, "planted columns")
