"""Parity of the LoSA-style block-wise path (sdattn_losa_*) with the fp64
oracle (oracle/losa.py), through the C ABI.

Each iteration is checked piece by piece:
  * page means of the cached keys against the oracle's pooling;
  * locality scores (fp64 on both sides) against the oracle's, and the Active
    list against the oracle's selection from its own scores, exact except for
    tokens within 1e-5 (relative) of the cut;
  * page scores (fp32) against the oracle's, element by element, and every kv
    head's page union against the oracle's per-row top-k of its own fp64 page
    scores: the union holds every page some row of the group must keep and
    only pages some row may keep (near-cut pages, within 1e-5 relative of a
    row's cut, may go either way);
  * Active rows of o / lse against the oracle's attention over (union pages +
    block) given the GPU's Active list and unions; Stable rows bit for bit
    unchanged.
Iterations chain: iteration 0 runs the dense form, later ones reuse the GPU's
previous outputs as o_prev (the oracle gets the same o_prev bytes).
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.losa as olosa
import sparse_bidirectional_attention_amd as sd
from gpu_util import check_out, check_topk_set, check_union_of_topk, host_inputs, say, to_dev, to_np
from workloads import tiny_random
from workloads.configs import LOSA_WORKLOADS, scaled
from workloads.generate import make_losa_base, make_losa_cache, make_losa_iteration

pytestmark = pytest.mark.gpu

SDAR = LOSA_WORKLOADS["losa_sdar8b_32k"]


def _problem(w):
    return sd.losa_problem(w.batch, w.q_heads, w.kv_heads, w.prefix_len, w.block_len, w.head_dim, w.page, w.n_active,
                           w.pages_per_query)


class _Run:
    """Device buffers of one block and its iterations."""

    def __init__(self, w, iters):
        self.w, self.p = w, _problem(w)
        base = make_losa_base(w)
        self.cache = make_losa_cache(w, base)
        self.iters = iters(base)
        self.kc, self.vc = to_dev(self.cache["k_cache"]), to_dev(self.cache["v_cache"])
        ws_bytes, self.cap = sd.sdattn_losa_workspace(self.p)
        self.ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
        B, Hq, Hkv = w.batch, w.q_heads, w.kv_heads
        self.n_pages = w.prefix_len // w.page
        self.kp = torch.empty(B, Hkv, self.n_pages, w.head_dim, dtype=torch.float32, device="cuda")
        sd.sdattn_losa_pool_pages(self.p, self.kc, self.kp)
        self.o = torch.empty(B, Hq, w.block_len, w.head_dim, dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty(B, Hq, w.block_len, dtype=torch.float32, device="cuda")
        self.active = torch.empty(B, w.n_active, dtype=torch.int32, device="cuda")
        self.upages = torch.full((B, Hkv, self.cap), -1, dtype=torch.int32, device="cuda")
        self.ucount = torch.empty(B, Hkv, dtype=torch.int32, device="cuda")
        self.loc = torch.empty(B, w.block_len, dtype=torch.float64, device="cuda")
        self.scores = torch.empty(B, Hq, w.n_active, self.n_pages, dtype=torch.float32, device="cuda")


def _dev(x):
    return {n: to_dev(a) for n, a in x.items()}


def _check_pool(run):
    kp_ref = olosa.pool_pages(run.cache["k_cache"], run.w.page)
    err = np.abs(to_np(run.kp) - kp_ref).max()
    assert err <= 1e-5 * max(1.0, np.abs(kp_ref).max()), f"page means max-abs {err:.3e}"


def _dense(run, x):
    w = run.w
    xd = _dev(x)
    sd.sdattn_losa_dense(run.p, xd["q"], run.kc, run.vc, xd["k_blk"], xd["v_blk"], run.o, run.lse, run.ws)
    torch.cuda.synchronize()
    o_ref, l_ref = olosa.losa_dense(x["q"], run.cache["k_cache"], run.cache["v_cache"], x["k_blk"], x["v_blk"])
    e = check_out(to_np(run.o), o_ref, to_np(run.lse), l_ref, "bf16", f"{w.name} dense")
    say(f"  dense: O max-abs {e[0]:.2e}")


def _step(run, x, x_prev, t, debug=True):
    w = run.w
    xd, xp = _dev(x), _dev(x_prev)
    o_prev, l_prev = host_inputs(run.o), to_np(run.lse)
    sd.sdattn_losa_step(run.p, xd["q"], xp["q"], run.kc, run.vc, run.kp, xd["k_blk"], xd["v_blk"], run.o, run.lse,
                        run.active, run.upages, run.ucount, run.ws, locality=run.loc if debug else None,
                        page_scores=run.scores if debug else None)
    torch.cuda.synchronize()
    active = run.active.cpu().numpy().astype(np.int64)
    counts = run.ucount.cpu().numpy()
    up = run.upages.cpu().numpy()
    unions = [[up[b, g, :counts[b, g]].astype(np.int64) for g in range(w.kv_heads)] for b in range(w.batch)]
    for b in range(w.batch):
        for g in range(w.kv_heads):
            assert 1 <= counts[b, g] <= run.cap and np.all(np.diff(unions[b][g]) > 0), f"union {b},{g} malformed"
    # The Active set and the page unions against the oracle's own fp64
    # locality and page scores: exact, except for candidates within CUT_REL
    # of a cut (LoSA, section 3, core principles).
    loc_ref = olosa.locality_scores(x["q"], x_prev["q"])
    for b in range(w.batch):
        check_topk_set(active[b], loc_ref[b], w.n_active, f"iteration {t} Active b={b}")
    kp_ref = olosa.pool_pages(run.cache["k_cache"], w.page)
    s_ref = olosa.page_scores(x["q"], active, kp_ref)
    G = w.q_heads // w.kv_heads
    n_near = 0
    for b in range(w.batch):
        for g in range(w.kv_heads):
            rows = s_ref[b, g * G:(g + 1) * G].reshape(-1, s_ref.shape[-1])
            n_near += check_union_of_topk(unions[b][g], rows, w.pages_per_query, f"iteration {t} union b={b} g={g}")
    if debug:
        loc = run.loc.cpu().numpy()
        np.testing.assert_allclose(loc, loc_ref, rtol=1e-12, atol=1e-300)
        s_gpu = run.scores.cpu().numpy().astype(np.float64)
        err = np.abs(s_gpu - s_ref).max()
        assert err <= 1e-5 * max(1.0, np.abs(s_ref).max()), f"page scores max-abs {err:.3e}"
    o_ref, l_ref = olosa.losa_attention(x["q"], run.cache["k_cache"], run.cache["v_cache"], x["k_blk"], x["v_blk"],
                                        active, unions, w.page, oracle.decode_bf16(o_prev), l_prev)
    o_new, l_new = host_inputs(run.o), to_np(run.lse)
    stable = np.ones((w.batch, w.block_len), dtype=bool)
    for b in range(w.batch):
        stable[b, active[b]] = False
        assert np.array_equal(o_new[b][:, stable[b]], o_prev[b][:, stable[b]]), f"iteration {t}: Stable O changed"
        assert np.array_equal(l_new[b][:, stable[b]], l_prev[b][:, stable[b]]), f"iteration {t}: Stable lse changed"
    e = check_out(oracle.decode_bf16(o_new), o_ref, l_new, l_ref, "bf16", f"{w.name} iteration {t}")
    say(f"  iteration {t}: active {active[0].tolist()} union sizes {counts.ravel().tolist()} near-cut pages {n_near} "
        f"O max-abs {e[0]:.2e}")


def _block(w, n_iter=4):
    say(f"losa {w.name}: B{w.batch} Hq{w.q_heads}/Hkv{w.kv_heads} Lp{w.prefix_len} Bs{w.block_len} d{w.head_dim} "
        f"page {w.page} active {w.n_active} pages/query {w.pages_per_query}")
    run = _Run(w, lambda base: [make_losa_iteration(w, t, base) for t in range(n_iter)])
    _check_pool(run)
    _dense(run, run.iters[0])
    for t in range(1, n_iter):
        _step(run, run.iters[t], run.iters[t - 1], t)
    return run


CASES = {
    "gqa4_l4096": dict(q_heads=8, kv_heads=2, prefix_len=4096, block_len=32, head_dim=128, page=16, n_active=8,
                       pages_per_query=4),
    "mha_b2_ragged": dict(batch=2, q_heads=4, kv_heads=4, prefix_len=3072, block_len=24, head_dim=64, page=32,
                          n_active=5, pages_per_query=3, n_moving=4),
    "gqa8_two_row_tiles": dict(q_heads=16, kv_heads=2, prefix_len=2048, block_len=64, head_dim=128, page=16,
                               n_active=16, pages_per_query=2, n_moving=12),
    "one_active_one_page": dict(q_heads=4, kv_heads=1, prefix_len=1024, block_len=8, head_dim=128, page=64,
                                n_active=1, pages_per_query=1, n_moving=1),
    "d64_rows_48_of_64": dict(q_heads=8, kv_heads=2, prefix_len=2048, block_len=32, head_dim=64, page=32,
                              n_active=12, pages_per_query=5, n_moving=10),
    "budget_over_64_pages": dict(q_heads=4, kv_heads=2, prefix_len=2048, block_len=16, head_dim=64, page=16,
                                 n_active=4, pages_per_query=100, n_moving=3),
    "pages_4096": dict(q_heads=2, kv_heads=1, prefix_len=65536, block_len=16, head_dim=64, page=16, n_active=4,
                       pages_per_query=16, n_moving=3),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_losa_block_matches_oracle(case):
    _block(scaled(SDAR, name=f"losa_{case}", **CASES[case]))


def test_losa_everything_active_full_budget_equals_dense():
    """All tokens Active and every page kept: the iteration must reproduce
    the dense attention of the new inputs."""
    w = scaled(SDAR, q_heads=4, kv_heads=2, prefix_len=1024, block_len=16, head_dim=128, page=16, n_active=16,
               pages_per_query=64, n_moving=16)
    run = _Run(w, lambda base: [make_losa_iteration(w, t, base) for t in range(2)])
    _dense(run, run.iters[0])
    _step(run, run.iters[1], run.iters[0], 1)
    assert np.all(run.ucount.cpu().numpy() == 64)
    o_ref, l_ref = olosa.losa_dense(run.iters[1]["q"], run.cache["k_cache"], run.cache["v_cache"],
                                    run.iters[1]["k_blk"], run.iters[1]["v_blk"])
    check_out(to_np(run.o), o_ref, to_np(run.lse), l_ref, "bf16", "all active, all pages")


def test_losa_random_inputs_and_no_debug_outputs():
    """Unstructured inputs (ties of the locality score impossible to plant by
    the generator), and the step without its optional outputs."""
    w = scaled(SDAR, q_heads=8, kv_heads=4, prefix_len=2048, block_len=32, head_dim=128, page=16, n_active=6,
               pages_per_query=5)

    def iters(base):
        out = []
        for t in range(3):
            r = tiny_random(700 + t, 1, 8, 4, 32, 128, dtype="bf16")
            out.append({"q": r["q"], "k_blk": r["k"], "v_blk": r["v"]})
        return out

    run = _Run(w, iters)
    _dense(run, run.iters[0])
    _step(run, run.iters[1], run.iters[0], 1, debug=False)
    _step(run, run.iters[2], run.iters[1], 2, debug=True)


def test_losa_full_size_block():
    """The block-wise workload at its full size (32K prefix, 32-token block,
    32/8 heads): dense iteration and three LoSA iterations, every row."""
    _block(SDAR, n_iter=4)


def test_losa_unchanged_queries_pick_lowest_indices():
    """q == q_prev: every locality score is 0 and the Active set is the first
    n_active tokens."""
    w = scaled(SDAR, q_heads=4, kv_heads=2, prefix_len=1024, block_len=16, head_dim=64, page=16, n_active=5,
               pages_per_query=2)
    run = _Run(w, lambda base: [make_losa_iteration(w, 0, base)] * 2)
    _dense(run, run.iters[0])
    _step(run, run.iters[1], run.iters[0], 1)
    assert run.active.cpu().tolist() == [[0, 1, 2, 3, 4]]
    assert np.all(run.loc.cpu().numpy() == 0.0)


def test_losa_step_captured_in_a_graph_replays_like_eager():
    """A LoSA iteration enqueues kernels only (the page bitmaps are cleared by a
    kernel, not a memset): captured once, replayed on new inputs copied into
    the captured buffers, it reproduces an eager run bit for bit, Active list
    and unions included."""
    w = scaled(SDAR, q_heads=8, kv_heads=2, prefix_len=4096, block_len=32, head_dim=128, page=16, n_active=8,
               pages_per_query=4)
    run = _Run(w, lambda base: [make_losa_iteration(w, t, base) for t in range(4)])
    xs = [_dev(x) for x in run.iters]
    sd.sdattn_losa_dense(run.p, xs[0]["q"], run.kc, run.vc, xs[0]["k_blk"], xs[0]["v_blk"], run.o, run.lse, run.ws)
    torch.cuda.synchronize()
    cur = {n: t.clone() for n, t in xs[1].items()}
    prev_q = xs[0]["q"].clone()
    o0, l0 = run.o.clone(), run.lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sd.sdattn_losa_step(run.p, cur["q"], prev_q, run.kc, run.vc, run.kp, cur["k_blk"], cur["v_blk"], run.o,
                            run.lse, run.active, run.upages, run.ucount, run.ws)
    for t in (1, 2, 3):
        for n in cur:
            cur[n].copy_(xs[t][n])
        prev_q.copy_(xs[t - 1]["q"])
        run.o.copy_(o0)
        run.lse.copy_(l0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in (run.o, run.lse, run.active, run.ucount, run.upages)]
        run.o.copy_(o0)
        run.lse.copy_(l0)
        sd.sdattn_losa_step(run.p, xs[t]["q"], xs[t - 1]["q"], run.kc, run.vc, run.kp, xs[t]["k_blk"],
                            xs[t]["v_blk"], run.o, run.lse, run.active, run.upages, run.ucount, run.ws)
        torch.cuda.synchronize()
        eager = (run.o, run.lse, run.active, run.ucount, run.upages)
        assert torch.equal(got[0].view(torch.int16), eager[0].view(torch.int16)), f"replay {t}: O"
        for a, b_, name in zip(got[1:], eager[1:], ("lse", "active", "union_count", "union_pages")):
            assert torch.equal(a, b_), f"replay {t}: {name}"
        say(f"  replay {t}: bit-identical to eager, active {run.active[0].tolist()}")
