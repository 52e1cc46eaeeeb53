"""Whole schedules through the C-ABI driver on the GPU, against the oracle.

Each step's action must equal the oracle's action table.  Every pattern the
driver selects is checked against the oracle's selection on that step's
inputs (exact up to near-cut candidates), and every step's output is checked
against the oracle's attention under the pattern in force (element by
element).  For the tiny fp32 workload the whole oracle schedule run is also
compared directly.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import sparse_bidirectional_attention_amd as sd
from gpu_util import check_out, check_topk_rows, csr_rows, host_inputs, say, to_dev, to_np
from test_gpu_select import _check_mass_rows
from workloads import WORKLOADS, make_base, make_step
from workloads.configs import scaled

pytestmark = pytest.mark.gpu

_hip = None


def _d2h(ptr, n, dtype=np.int32):
    """Copy n elements from a raw device pointer (borrowed from the handle)."""
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    out = np.empty(n, dtype=dtype)
    assert _hip.hipMemcpy(out.ctypes.data, ptr, out.nbytes, 2) == 0  # device to host
    return out


def _desc(w, split_rows=False):
    sel = sd.SEL_KINDS[w.selector]
    budget = sd.topk_budget(w.keep_frac) if w.budget == "topk" else sd.mass_budget(w.mass, w.max_mean_density)
    return sd.schedule_desc(w.total_steps, w.dense_steps, w.select_step, w.refresh_interval, list(w.refresh_steps),
                            w.refresh_dense, sel, w.block, w.block, budget, w.column_keep_frac,
                            w.probe_interval, w.min_overlap, split_rows)


def _run_and_check(w, split_rows=False):
    base = make_base(w)
    p = sd.problem(w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.dtype)
    acts_ref = oracle.schedule_actions(w.total_steps, w.dense_steps, w.select_step, w.refresh_interval,
                                       w.refresh_steps, w.refresh_dense)
    h = sd.sdattn_schedule_create(p, _desc(w, split_rows))
    nqb = -(-w.seq_len // w.block)
    rows = w.batch * w.q_heads * nqb
    kcol = oracle.count_from_fraction(w.column_keep_frac, w.seq_len) if w.selector == "columns" else 0
    pattern = None
    outs = []
    try:
        for t in range(w.total_steps):
            xh = make_step(w, t, base)
            x = {n: to_dev(a) for n, a in xh.items()}
            o = torch.empty_like(x["q"])
            lse = torch.empty(x["q"].shape[:3], dtype=torch.float32, device="cuda")
            act = sd.sdattn_schedule_action(h, t)
            assert act == acts_ref[t]
            sd.sdattn_schedule_step(h, t, x["q"], x["k"], x["v"], o, lse)
            torch.cuda.synchronize()
            hq, hk, hv = (host_inputs(x[n]) for n in "qkv")
            if act in ("DENSE", "DENSE_SELECT"):
                ro, rl = oracle.dense_attention(hq, hk, hv)
            if act in ("DENSE_SELECT", "SELECT_SPARSE"):
                rp_ptr, ci_ptr, cap = sd.sdattn_schedule_mask(h)
                if w.selector == "blocks":
                    rp = _d2h(rp_ptr, rows + 1)
                    ci = _d2h(ci_ptr, int(rp[-1]))
                    A4 = oracle.pooled_mass(hq, hk, w.block, w.block)
                    A = A4.reshape(rows, -1)
                    if w.budget == "topk":
                        check_topk_rows(csr_rows(rp, ci), A, oracle.count_from_fraction(w.keep_frac, A.shape[1]))
                    else:
                        _, _, tau = oracle.select_mass_cap(A4, w.mass, w.max_mean_density)
                        _check_mass_rows(rp, ci, A, tau, w.mass, w.max_mean_density)
                    pattern = (rp, ci)
                else:
                    cols = _d2h(ci_ptr, w.batch * w.kv_heads * kcol).reshape(w.batch, w.kv_heads, kcol)
                    C = oracle.column_scores(hq, hk, oracle.dense_attention(hq, hk, hv)[1])
                    for b in range(w.batch):
                        check_topk_rows(cols[b], C[b], kcol, "columns")
                    pattern_next = cols
            if act in ("SELECT_SPARSE", "SPARSE"):
                if w.selector == "blocks":
                    ro, rl = oracle.block_sparse_attention(hq, hk, hv, pattern[0], pattern[1], w.block, w.block)
                else:
                    ro, rl = oracle.column_sparse_attention(hq, hk, hv, pattern)
            if w.selector == "columns" and act == "DENSE_SELECT":
                pattern = pattern_next  # a column pattern applies from the next step
            check_out(to_np(o), ro, to_np(lse), rl, w.dtype, f"step {t} {act}")
            outs.append((act, to_np(o), to_np(lse)))
        stats, last = sd.sdattn_schedule_stats(h)
    finally:
        sd.sdattn_schedule_destroy(h)
    return outs, stats, last, base


def test_tiny_fp32_schedule_every_step():
    w = WORKLOADS["tiny_fp32_h4_l512"]
    say(f"schedule {w.name}")
    outs, stats, last, base = _run_and_check(w)
    assert stats == {"DENSE": 0, "DENSE_SELECT": 1, "SELECT_SPARSE": 0, "SPARSE": 3} and last == 0
    ref = oracle.run_schedule(w, lambda t: make_step(w, t, base))
    for (act, o, lse), r in zip(outs, ref):
        check_out(o, r["o"], lse, r["lse"], "f32", f"oracle schedule step {r['step']}")


def test_small_mass_refresh_schedule_bf16():
    w = scaled(WORKLOADS["llada8b_8k"], seq_len=1024, q_heads=4, kv_heads=4, total_steps=7, refresh_interval=3,
               max_mean_density=0.3)
    say("schedule mass+cap scaled L=1024 T=7")
    _, stats, last, _ = _run_and_check(w)
    assert stats["SELECT_SPARSE"] == 2 and last == 6


def test_small_uncapped_mass_schedule_with_split_rows_bf16():
    """A mass budget with no cap (head-adaptive: the heads without planted
    structure keep most blocks, the others few) and split rows: the long rows
    are cut and merged, and every step still matches the oracle under the
    pattern in force."""
    w = scaled(WORKLOADS["llada8b_8k"], seq_len=1024, q_heads=4, kv_heads=4, total_steps=7, refresh_interval=3,
               max_mean_density=1.0)
    say("schedule uncapped mass, split rows, scaled L=1024 T=7")
    _, stats, last, _ = _run_and_check(w, split_rows=True)
    assert stats["SELECT_SPARSE"] == 2 and last == 6


def test_small_topk_warmup_schedule_bf16():
    w = scaled(WORKLOADS["sparsed_64k"], seq_len=2048, q_heads=4, kv_heads=4, total_steps=6, dense_steps=2,
               select_step=2)
    say("schedule topk warm-up scaled L=2048 T=6")
    _, stats, last, _ = _run_and_check(w)
    assert stats == {"DENSE": 2, "DENSE_SELECT": 0, "SELECT_SPARSE": 1, "SPARSE": 3} and last == 2


def test_small_column_schedule_gqa():
    w = scaled(WORKLOADS["pulsecol_dream7b_16k"], seq_len=1024, q_heads=6, kv_heads=2, total_steps=5,
               refresh_steps=(3,), n_stripe_columns=20)
    say("schedule columns scaled L=1024 T=5")
    _, stats, last, _ = _run_and_check(w)
    assert stats == {"DENSE": 0, "DENSE_SELECT": 2, "SELECT_SPARSE": 0, "SPARSE": 3} and last == 3
