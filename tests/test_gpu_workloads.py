"""Full-size parity on the five workloads, through the schedule driver (the
launch configuration bench.py times).

Masks are checked in full (top-k / mass-cap rules, exact up to near-cut
candidates).  Outputs are checked element by element on sampled query rows
or query blocks (always including the first and the last), which the fp64
oracle computes one by one: dense rows against all keys, sparse rows in
gather form under the GPU's pattern.  The checked steps follow each
schedule; skipped steps never select, so the pattern in force is the one a
full run would have.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

import oracle
import sparse_bidirectional_attention_amd as sd
from gpu_util import check_out, check_topk_rows, csr_rows, host_inputs, say, to_dev, to_np
from test_gpu_schedule import _d2h, _desc
from test_gpu_select import _check_mass_rows
from workloads import WORKLOADS, make_base, make_step

pytestmark = pytest.mark.gpu


def _sample(n, k):
    s = np.unique(np.concatenate([np.linspace(0, n - 1, k).astype(int), [0, n - 1]]))
    return s


def _check_column_groups(w, xh, cols, kcol, groups):
    """The column selection of each kv group in `groups` against the top-kcol
    of the oracle's fp64 column scores, which read the oracle's own dense
    log-sum-exp (PulseCol, Abstract).  The groups are independent, so the
    oracle runs them on a thread pool (numpy's ufuncs and BLAS release the
    interpreter lock); the results are the plain serial ones."""
    G = w.q_heads // w.kv_heads

    def one(g):
        sl = slice(g * G, (g + 1) * G)
        _, rl = oracle.dense_attention(xh["q"][:, sl], xh["k"][:, g:g + 1], xh["v"][:, g:g + 1])
        C = oracle.column_scores(xh["q"][:, sl], xh["k"][:, g:g + 1], rl)
        return check_topk_rows(cols[0, g:g + 1], C[0], kcol, f"columns g={g}")

    if len(groups) <= 1:
        return [one(g) for g in groups]
    with threadpool_limits(limits=max(1, (os.cpu_count() or 4) // len(groups)), user_api="blas"):
        with ThreadPoolExecutor(len(groups)) as ex:
            return list(ex.map(one, groups))


def _run_steps(w, steps, n_qblocks=8, n_rows=32, col_groups=None):
    """col_groups: for a column workload, {step: [kv groups whose selection is
    checked]}; None checks every group at every selection step."""
    base = make_base(w)
    p = sd.problem(w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.dtype)
    acts = oracle.schedule_actions(w.total_steps, w.dense_steps, w.select_step, w.refresh_interval,
                                   w.refresh_steps, w.refresh_dense)
    h = sd.sdattn_schedule_create(p, _desc(w))
    L, H = w.seq_len, w.q_heads
    nqb = -(-L // w.block)
    rows = w.batch * H * nqb
    kcol = oracle.count_from_fraction(w.column_keep_frac, L) if w.selector == "columns" else 0
    pattern, pending = None, None
    try:
        for t in steps:
            act = acts[t]
            say(f"{w.name} step {t} {act}")
            xh = make_step(w, t, base)
            x = {n: to_dev(a) for n, a in xh.items()}
            o = torch.empty_like(x["q"])
            lse = torch.empty(x["q"].shape[:3], dtype=torch.float32, device="cuda")
            assert sd.sdattn_schedule_action(h, t) == act
            sd.sdattn_schedule_step(h, t, x["q"], x["k"], x["v"], o, lse)
            torch.cuda.synchronize()
            og, lg = to_np(o), to_np(lse)
            del x, o, lse
            if act in ("DENSE_SELECT", "SELECT_SPARSE"):
                rp_ptr, ci_ptr, _ = sd.sdattn_schedule_mask(h)
                if w.selector == "blocks":
                    rp = _d2h(rp_ptr, rows + 1)
                    ci = _d2h(ci_ptr, int(rp[-1]))
                    A4 = oracle.pooled_mass(xh["q"], xh["k"], w.block, w.block)
                    A = A4.reshape(rows, -1)
                    if w.budget == "topk":
                        n_ex = check_topk_rows(csr_rows(rp, ci), A, oracle.count_from_fraction(w.keep_frac, nqb))
                    else:
                        _, _, tau = oracle.select_mass_cap(A4, w.mass, w.max_mean_density)
                        _check_mass_rows(rp, ci, A, tau, w.mass, w.max_mean_density)
                        n_ex = None
                    say(f"  mask: nnz={rp[-1]} density={rp[-1] / A.size:.4f} exempt rows={n_ex}")
                    pattern = (rp, ci)
                else:
                    cols = _d2h(ci_ptr, w.batch * w.kv_heads * kcol).reshape(w.batch, w.kv_heads, kcol)
                    groups = list(range(w.kv_heads)) if col_groups is None else col_groups.get(t, [])
                    for g, n_ex in zip(groups, _check_column_groups(w, xh, cols, kcol, groups)):
                        say(f"  columns g={g}: exempt={n_ex}")
                    pending = cols
            # outputs on samples
            if act in ("DENSE", "DENSE_SELECT"):
                r = _sample(L, n_rows)
                ro, rl = oracle.dense_attention(xh["q"], xh["k"], xh["v"], rows=r)
                check_out(og[:, :, r], ro, lg[:, :, r], rl, w.dtype, f"step {t} dense rows")
            elif w.selector == "blocks":
                qb = _sample(nqb, n_qblocks)
                ro, rl = oracle.block_sparse_attention(xh["q"], xh["k"], xh["v"], pattern[0], pattern[1], w.block,
                                                       w.block, qblocks=qb)
                toks = np.concatenate([np.arange(I * w.block, min(L, (I + 1) * w.block)) for I in qb])
                e = check_out(og[:, :, toks], ro, lg[:, :, toks], rl, w.dtype, f"step {t} sparse blocks")
                say(f"  O max-abs {e[0]:.2e} mean-abs {e[1]:.2e}")
            else:
                r = _sample(L, n_rows)
                ro, rl = oracle.column_sparse_attention(xh["q"], xh["k"], xh["v"], pattern, rows=r)
                e = check_out(og[:, :, r], ro, lg[:, :, r], rl, w.dtype, f"step {t} column rows")
                say(f"  O max-abs {e[0]:.2e} mean-abs {e[1]:.2e}")
            if act == "DENSE_SELECT" and w.selector == "columns":
                pattern = pending
    finally:
        sd.sdattn_schedule_destroy(h)


def test_llada8b_8k_mass_cap_refresh():
    _run_steps(WORKLOADS["llada8b_8k"], [0, 1, 31, 32, 33, 224, 255], n_qblocks=16)


def test_sparsed_32k_topk():
    _run_steps(WORKLOADS["sparsed_32k"], [25, 26, 127], n_qblocks=16)


def test_sparsed_64k_topk():
    _run_steps(WORKLOADS["sparsed_64k"], [204, 205, 1023], n_qblocks=8, n_rows=16)


def test_pulsecol_16k_columns_first_selection():
    """Step 0 selects the columns of all four kv groups: every group's
    selection against the oracle, then the sparse steps that reuse it."""
    _run_steps(WORKLOADS["pulsecol_dream7b_16k"], [0, 1, 63], n_rows=64, col_groups={0: [0, 1, 2, 3]})


def test_pulsecol_16k_columns_refresh_64():
    """The refresh at step 64 selects from its own dense pass: kv group 1's
    selection against the oracle, then the sparse step that reuses it."""
    _run_steps(WORKLOADS["pulsecol_dream7b_16k"], [64, 65], n_rows=64, col_groups={64: [1]})


def test_pulsecol_16k_columns_refresh_128():
    """The refresh at step 128: kv group 2's selection against the oracle,
    then sparse steps up to the schedule's last."""
    _run_steps(WORKLOADS["pulsecol_dream7b_16k"], [128, 129, 191], n_rows=64, col_groups={128: [2]})
