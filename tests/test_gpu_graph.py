"""Schedule steps captured in a HIP graph (through torch.cuda.graph) and
replayed, against the same steps run eagerly.

A step enqueues kernels only (no memset, copy, allocation or host wait), so a
caller that cannot afford per-step launches can capture steps once and replay
them.  Each replay runs on new input contents (copied into the captured
buffers, with eager work and a synchronisation between replays) and must
reproduce the eager outputs bit for bit: same kernels, same inputs.  A
captured probe step must also take the same decisions as the eager one.
"""

import numpy as np
import pytest
import torch

import sparse_bidirectional_attention_amd as sd
from gpu_util import say, to_dev
from test_gpu_probe import _d2h
from workloads import WORKLOADS, make_base, make_step
from workloads.configs import scaled

pytestmark = pytest.mark.gpu


def _desc(w, split_rows=False):
    budget = sd.topk_budget(w.keep_frac) if w.budget == "topk" else sd.mass_budget(w.mass, w.max_mean_density)
    return sd.schedule_desc(w.total_steps, w.dense_steps, w.select_step, w.refresh_interval, list(w.refresh_steps),
                            w.refresh_dense, sd.SEL_KINDS[w.selector], w.block, w.block, budget, w.column_keep_frac,
                            w.probe_interval, w.min_overlap, split_rows)


def _inputs(w, base, t):
    return {n: to_dev(a) for n, a in make_step(w, t, base).items()}


@pytest.mark.parametrize("split_rows", [False, True])
def test_captured_sparse_steps_replay_like_eager_ones(split_rows):
    """Also with split rows: a captured step is then the forward over the split
    plan and the merge of the cut rows (at this size rows of more than 4 kept
    blocks are cut)."""
    w = scaled(WORKLOADS["llada8b_8k"], seq_len=2048, q_heads=4, kv_heads=4, total_steps=8, refresh_interval=0,
               max_mean_density=0.3)
    say(f"graph: capture 3 sparse steps, L=2048 mass budget, split rows {split_rows}")
    p = sd.problem(w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.dtype)
    base = make_base(w)
    h = sd.sdattn_schedule_create(p, _desc(w, split_rows))
    try:
        x0 = _inputs(w, base, 0)
        o0 = torch.empty_like(x0["q"])
        sd.sdattn_schedule_step(h, 0, x0["q"], x0["k"], x0["v"], o0)  # DENSE_SELECT: the pattern
        torch.cuda.synchronize()
        # static buffers for steps 1..3 (SPARSE), captured once
        xs = [_inputs(w, base, t) for t in (1, 2, 3)]
        os_ = [torch.empty_like(x["q"]) for x in xs]
        ls = [torch.empty(x["q"].shape[:3], dtype=torch.float32, device="cuda") for x in xs]
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):  # one eager warm-up on the capture stream
            for i, t in enumerate((1, 2, 3)):
                sd.sdattn_schedule_step(h, t, xs[i]["q"], xs[i]["k"], xs[i]["v"], os_[i], ls[i])
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i, t in enumerate((1, 2, 3)):
                sd.sdattn_schedule_step(h, t, xs[i]["q"], xs[i]["k"], xs[i]["v"], os_[i], ls[i])
        for rep, ts in enumerate([(1, 2, 3), (4, 5, 6), (7, 2, 5)]):
            for i, t in enumerate(ts):  # new contents into the captured buffers
                xt = _inputs(w, base, t)
                for n in "qkv":
                    xs[i][n].copy_(xt[n])
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            got = [(o.clone(), l.clone()) for o, l in zip(os_, ls)]
            # eager on the same inputs, into other buffers
            for i, t in enumerate(ts):
                oe = torch.empty_like(os_[i])
                le = torch.empty_like(ls[i])
                sd.sdattn_schedule_step(h, 1, xs[i]["q"], xs[i]["k"], xs[i]["v"], oe, le)
                torch.cuda.synchronize()
                assert torch.equal(oe.view(torch.int16), got[i][0].view(torch.int16)), f"replay {rep} step {t}: O"
                assert torch.equal(le, got[i][1]), f"replay {rep} step {t}: lse"
            say(f"  replay {rep}: bit-identical to eager")
    finally:
        torch.cuda.synchronize()
        sd.sdattn_schedule_destroy(h)


@pytest.mark.parametrize("budget", ["topk", "mass"])
def test_captured_probe_step_decides_like_eager(budget):
    """A probe step (selection, overlap counts cleared by a kernel, adoption,
    attention) captured once: replayed on a drifting input it keeps the
    pattern, on unrelated inputs it adopts the probe; the outputs and the
    probe record match an eager handle run on the same sequence.  The
    capped-mass selection adds the radix-select kernels to the graph."""
    w = scaled(WORKLOADS["sparsed_64k"], seq_len=2048, q_heads=4, kv_heads=4, total_steps=6, dense_steps=1,
               select_step=1, keep_frac=0.25, probe_interval=1, min_overlap=0.6)
    if budget == "mass":
        w = scaled(w, budget="mass", mass=0.95, max_mean_density=0.25)
    say(f"graph: capture a probe step, L=2048 {budget}")
    p = sd.problem(w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.dtype)
    base, other = make_base(w), make_base(scaled(w, wid=103))
    seq = [(base, 2), (other, 3), (other, 4)]  # keep, adopt, keep
    hg = sd.sdattn_schedule_create(p, _desc(w))
    he = sd.sdattn_schedule_create(p, _desc(w))
    try:
        for h in (hg, he):
            for t in (0, 1):  # DENSE, SELECT_SPARSE
                x = _inputs(w, base, t)
                sd.sdattn_schedule_step(h, t, x["q"], x["k"], x["v"], torch.empty_like(x["q"]))
        torch.cuda.synchronize()
        xb = _inputs(w, base, 2)
        ob = torch.empty_like(xb["q"])
        lb = torch.empty(xb["q"].shape[:3], dtype=torch.float32, device="cuda")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sd.sdattn_schedule_step(hg, 2, xb["q"], xb["k"], xb["v"], ob, lb)
        for i, (src, t) in enumerate(seq):
            xt = _inputs(w, src, t)
            for n in "qkv":
                xb[n].copy_(xt[n])
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            oe = torch.empty_like(ob)
            le = torch.empty_like(lb)
            sd.sdattn_schedule_step(he, 2 + i, xt["q"], xt["k"], xt["v"], oe, le)
            torch.cuda.synchronize()
            sg, se = sd.sdattn_schedule_probe_stats(hg), sd.sdattn_schedule_probe_stats(he)
            say(f"  replay {i}: graph {sg} eager {se}")
            assert sg[1:] == se[1:] and sg[0] == se[0] == i + 1
            assert torch.equal(oe.view(torch.int16), ob.view(torch.int16)) and torch.equal(le, lb)
        if budget == "topk":
            assert sd.sdattn_schedule_probe_stats(hg)[1] == 1  # exactly the unrelated inputs were adopted
        rg, cg, _ = sd.sdattn_schedule_mask(hg)
        re_, ce, _ = sd.sdattn_schedule_mask(he)
        rows = w.q_heads * (w.seq_len // w.block)
        a, b = _d2h(rg, rows + 1), _d2h(re_, rows + 1)
        np.testing.assert_array_equal(a, b)
        np.testing.assert_array_equal(_d2h(cg, int(a[-1])), _d2h(ce, int(a[-1])))
    finally:
        torch.cuda.synchronize()
        sd.sdattn_schedule_destroy(hg)
        sd.sdattn_schedule_destroy(he)
