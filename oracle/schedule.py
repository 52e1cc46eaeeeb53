"""Step schedule of the denoising loop — test infrastructure only.

SparseD abstract: full attention in the early steps, then a head-specific
pattern computed once and reused at every later step.  Step-dLLM abstract:
the block mask is refreshed at anchor steps and reused within each interval.
PulseCol abstract: the column pattern is identified at an early step and
refreshed only at a few intermediate steps.

Adaptive anchors (block patterns).  Step-dLLM's abstract observes that
attention patterns hold only locally across steps and change abruptly at
some transitions.  Reading: between anchors the pooled selector is rerun
every `probe_interval` steps (a probe); the probe B replaces the cached
pattern A when their overlap J = |A n B| / |A u B|, over (row, block)
pairs, is below `min_overlap` (J = 1 when both are empty).

Action of step t, with S = {select_step} u {select_step + m * interval, m >= 1}
u refresh_steps (steps below total_steps):
  t in S     : DENSE_SELECT if t < dense_steps or (refresh_dense and t > select_step),
               else SELECT_SPARSE;
  t not in S : DENSE if t < dense_steps; else PROBE_SPARSE if probe_interval > 0,
               t > select_step and (t - select_step) mod probe_interval == 0;
               else SPARSE.
SELECT_SPARSE selects from the step's own Q/K and then attends with the new
mask.  DENSE_SELECT attends densely; a block pattern is selected from the
step's Q/K, a column pattern from the dense pass's log-sum-exp; either
applies from the next sparse step on.
"""

import numpy as np

from .attention import block_sparse_attention, column_sparse_attention, dense_attention
from .select import (
    column_scores,
    count_from_fraction,
    exact_block_mass,
    pooled_mass,
    select_columns,
    select_mass_cap,
    select_topk,
)

ACTIONS = ("DENSE", "DENSE_SELECT", "SELECT_SPARSE", "SPARSE", "PROBE_SPARSE")


def select_steps(total_steps, select_step, refresh_interval=0, refresh_steps=()):
    s = {select_step}
    if refresh_interval > 0:
        s.update(range(select_step + refresh_interval, total_steps, refresh_interval))
    s.update(refresh_steps)
    return {t for t in s if 0 <= t < total_steps}


def schedule_actions(total_steps, dense_steps, select_step, refresh_interval=0,
                     refresh_steps=(), refresh_dense=False, probe_interval=0):
    if select_step > dense_steps:
        raise ValueError("the first sparse step would have no pattern")
    S = select_steps(total_steps, select_step, refresh_interval, refresh_steps)
    acts = []
    for t in range(total_steps):
        if t in S:
            dense = t < dense_steps or (refresh_dense and t > select_step)
            acts.append("DENSE_SELECT" if dense else "SELECT_SPARSE")
        elif t < dense_steps:
            acts.append("DENSE")
        elif probe_interval > 0 and t > select_step and (t - select_step) % probe_interval == 0:
            acts.append("PROBE_SPARSE")
        else:
            acts.append("SPARSE")
    return acts


def _pairs(row_ptr, col_idx):
    rp = np.asarray(row_ptr, dtype=np.int64)
    ci = np.asarray(col_idx, dtype=np.int64)
    return {(r, int(c)) for r in range(len(rp) - 1) for c in ci[rp[r]:rp[r + 1]]}


def mask_overlap(row_ptr_a, col_idx_a, row_ptr_b, col_idx_b):
    """(|A n B|, |A|, |B|) of two CSR block patterns over the same rows,
    each taken as a set of (row, block) pairs."""
    A = _pairs(row_ptr_a, col_idx_a)
    B = _pairs(row_ptr_b, col_idx_b)
    return len(A & B), len(A), len(B)


def overlap_ratio(inter, na, nb):
    """J = |A n B| / |A u B| from the counts; 1 when both patterns are empty."""
    union = na + nb - inter
    return 1.0 if union == 0 else inter / union


def probe_adopts(inter, na, nb, min_overlap):
    """A probe replaces the cached pattern when its overlap is below min_overlap."""
    return overlap_ratio(inter, na, nb) < min_overlap


def run_schedule(w, step_inputs, steps=None):
    """Run a whole schedule of workload `w` (small shapes only).

    step_inputs(t) -> dict(q, k, v) for step t.  Returns a list, per step, of
    dict(action, o, lse, pattern) where pattern is (row_ptr, col_idx) for
    blocks (pooled or exact) or col_idx for columns (the pattern in force
    after the step; a DENSE_SELECT step's pattern applies from the next); a
    probe step also gives the probe's counts (|A n B|, |A|, |B|) and whether
    it was adopted.
    """
    acts = schedule_actions(w.total_steps, w.dense_steps, w.select_step, w.refresh_interval,
                            w.refresh_steps, w.refresh_dense, w.probe_interval)
    steps = range(w.total_steps) if steps is None else steps
    pattern = None
    out = []
    for t in range(w.total_steps):
        a = acts[t]
        x = step_inputs(t)
        q, k, v = x["q"], x["k"], x["v"]
        o = lse = None
        probe = None
        if w.selector == "blocks_exact":
            # the exact block mass needs the dense pass's log-sum-exp: every
            # selection step is dense; the pattern applies from the next step
            if a in ("DENSE", "DENSE_SELECT"):
                o, lse = dense_attention(q, k, v)
                if a == "DENSE_SELECT":
                    A = exact_block_mass(q, k, lse, w.block, w.block)
                    if w.budget == "topk":
                        pattern = select_topk(A, w.keep_frac)
                    else:
                        rp, ci, _ = select_mass_cap(A, w.mass, w.max_mean_density)
                        pattern = (rp, ci)
            else:
                o, lse = block_sparse_attention(q, k, v, pattern[0], pattern[1], w.block, w.block)
        elif w.selector == "blocks":
            if a in ("DENSE_SELECT", "SELECT_SPARSE", "PROBE_SPARSE"):
                A = pooled_mass(q, k, w.block, w.block)
                if w.budget == "topk":
                    new = select_topk(A, w.keep_frac)
                else:
                    rp, ci, _ = select_mass_cap(A, w.mass, w.max_mean_density)
                    new = (rp, ci)
                if a == "PROBE_SPARSE":
                    counts = mask_overlap(pattern[0], pattern[1], new[0], new[1])
                    adopted = probe_adopts(*counts, w.min_overlap)
                    probe = {"counts": counts, "adopted": adopted}
                    if adopted:
                        pattern = new
                else:
                    pattern = new
            if a in ("DENSE", "DENSE_SELECT"):
                o, lse = dense_attention(q, k, v)
            else:
                o, lse = block_sparse_attention(q, k, v, pattern[0], pattern[1], w.block, w.block)
        else:
            if a in ("DENSE", "DENSE_SELECT"):
                o, lse = dense_attention(q, k, v)
                if a == "DENSE_SELECT":
                    kcol = count_from_fraction(w.column_keep_frac, np.asarray(k).shape[2])
                    pattern = select_columns(column_scores(q, k, lse), kcol)
            else:
                o, lse = column_sparse_attention(q, k, v, pattern)
        if t in steps:
            out.append({"step": t, "action": a, "o": o, "lse": lse, "pattern": pattern, "probe": probe})
    return out
