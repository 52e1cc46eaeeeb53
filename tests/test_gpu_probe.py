"""Adaptive anchors on the GPU, through the C ABI.

* sdattn_mask_overlap against the oracle's set arithmetic: the counts
  (|A n B|, |A|, |B|) are integers and must match exactly, from empty
  patterns up to the 64K top-5% mask shape (16,384 rows of 26 blocks).
* Schedules with probes through the driver: each probe's decision must equal
  the oracle's (the probe's overlap with the cached pattern, against the
  threshold), a kept pattern must stay bit-identical, an adopted one must be
  the step's selection (exact up to near-cut candidates), and every step's
  output must match the oracle's attention under the pattern in force.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import sparse_bidirectional_attention_amd as sd
from gpu_util import check_out, check_topk_rows, csr_rows, dev_csr, host_inputs, say, to_dev, to_np
from workloads import WORKLOADS, make_base, make_step
from workloads.configs import scaled

pytestmark = pytest.mark.gpu

_hip = None


def _d2h(ptr, n):
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    out = np.empty(n, dtype=np.int32)
    if n:
        assert _hip.hipMemcpy(out.ctypes.data, ptr, out.nbytes, 2) == 0
    return out


def _rand_csr(rng, rows, nkb, density):
    keep = np.ones((rows, nkb), bool) if density >= 1 else rng.random((rows, nkb)) < density
    rp = np.zeros(rows + 1, np.int32)
    rp[1:] = np.cumsum(keep.sum(1))
    return rp, np.nonzero(keep)[1].astype(np.int32)


def _topk_csr(rng, rows, nkb, k):
    """k distinct blocks per row, ascending: the shape a top-k selection writes."""
    ci = np.sort(np.argsort(rng.random((rows, nkb)), axis=1)[:, :k], axis=1)
    return (np.arange(rows + 1) * k).astype(np.int32), ci.astype(np.int32).reshape(-1)


def _gpu_counts(rows, a, b):
    ra, ca = dev_csr(*a)
    rb, cb = dev_csr(*b)
    counts = torch.full((3,), -7, dtype=torch.int64, device="cuda")  # overwritten, not accumulated
    sd.sdattn_mask_overlap(rows, ra, ca, rb, cb, counts)
    torch.cuda.synchronize()
    return tuple(int(x) for x in counts.cpu())


# (rows, nKB, density of A, density of B): single entries, empty and full rows,
# rows longer than a wave (1024 blocks), a ragged last workgroup
CASES = [(1, 1, 1.0, 1.0), (1, 8, 0.0, 0.5), (5, 8, 0.0, 0.0), (7, 8, 0.5, 0.5), (33, 64, 0.2, 0.9),
         (1000, 128, 0.1, 0.1), (257, 1024, 1.0, 0.3), (300, 1024, 0.05, 1.0), (4097, 128, 0.1, 0.12)]


@pytest.mark.parametrize("case", CASES)
def test_mask_overlap_matches_oracle(case):
    rows, nkb, da, db = case
    say(f"mask overlap rows={rows} nKB={nkb} densities {da}/{db}")
    rng = np.random.default_rng(rows * 131 + nkb)
    a = _rand_csr(rng, rows, nkb, da)
    b = _rand_csr(rng, rows, nkb, db)
    assert _gpu_counts(rows, a, b) == oracle.mask_overlap(*a, *b)
    assert _gpu_counts(rows, b, a) == oracle.mask_overlap(*b, *a)
    assert _gpu_counts(rows, a, a) == oracle.mask_overlap(*a, *a)


def test_mask_overlap_of_no_rows():
    counts = torch.full((3,), -7, dtype=torch.int64, device="cuda")
    sd.sdattn_mask_overlap(0, None, None, None, None, counts)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0, 0, 0]


def test_mask_overlap_at_the_64k_mask_shape():
    """16,384 rows of 26 of 512 blocks: unrelated patterns, and a pattern with
    about a third of every row's blocks replaced."""
    say("mask overlap 64K shape")
    rng = np.random.default_rng(64)
    rows, nkb, k = 16384, 512, 26
    a = _topk_csr(rng, rows, nkb, k)
    b = _topk_csr(rng, rows, nkb, k)
    assert _gpu_counts(rows, a, b) == oracle.mask_overlap(*a, *b)
    # moved: keep 17 of each row's blocks of A, take 9 more from B's row that are not in it
    ra = a[1].reshape(rows, k)
    rb = b[1].reshape(rows, k)
    moved = []
    for r in range(rows):
        keep = set(ra[r][:17].tolist())
        extra = [x for x in rb[r].tolist() + list(range(nkb)) if x not in keep]
        moved.append(sorted(keep | set(extra[:k - 17])))
    c = (a[0], np.asarray(moved, np.int32).reshape(-1))
    got = _gpu_counts(rows, a, c)
    assert got == oracle.mask_overlap(*a, *c)
    assert got[0] >= 17 * rows


def _probe_desc(w):
    budget = sd.topk_budget(w.keep_frac) if w.budget == "topk" else sd.mass_budget(w.mass, w.max_mean_density)
    return sd.schedule_desc(w.total_steps, w.dense_steps, w.select_step, w.refresh_interval, list(w.refresh_steps),
                            w.refresh_dense, sd.SDATTN_SEL_BLOCKS, w.block, w.block, budget, 0.0,
                            w.probe_interval, w.min_overlap)


def _run_probe_schedule(w, inputs):
    """Runs the schedule on the GPU; checks every step against the oracle.
    Returns the decisions [(step, adopted, overlap)]."""
    p = sd.problem(w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.dtype)
    acts = oracle.schedule_actions(w.total_steps, w.dense_steps, w.select_step, w.refresh_interval,
                                   w.refresh_steps, w.refresh_dense, w.probe_interval)
    rows = w.batch * w.q_heads * (-(-w.seq_len // w.block))
    h = sd.sdattn_schedule_create(p, _probe_desc(w))
    pattern = None
    decisions = []
    n_adopted = 0
    try:
        for t in range(w.total_steps):
            xh = inputs(t)
            x = {n: to_dev(a) for n, a in xh.items()}
            o = torch.empty_like(x["q"])
            lse = torch.empty(x["q"].shape[:3], dtype=torch.float32, device="cuda")
            act = sd.sdattn_schedule_action(h, t)
            assert act == acts[t]
            sd.sdattn_schedule_step(h, t, x["q"], x["k"], x["v"], o, lse)
            torch.cuda.synchronize()
            hq, hk, hv = (host_inputs(x[n]) for n in "qkv")
            if act in ("DENSE_SELECT", "SELECT_SPARSE", "PROBE_SPARSE"):
                rp_ptr, ci_ptr, _ = sd.sdattn_schedule_mask(h)
                rp = _d2h(rp_ptr, rows + 1)
                now = (rp, _d2h(ci_ptr, int(rp[-1])))
                A4 = oracle.pooled_mass(hq, hk, w.block, w.block)
                sel = oracle.select_topk(A4, w.keep_frac)
                k = oracle.count_from_fraction(w.keep_frac, A4.shape[-1])
                if act == "PROBE_SPARSE":
                    ref_counts = oracle.mask_overlap(pattern[0], pattern[1], sel[0], sel[1])
                    ref_adopt = oracle.probe_adopts(*ref_counts, w.min_overlap)
                    n_probes, adopted, j = sd.sdattn_schedule_probe_stats(h)
                    new_adopt = adopted > n_adopted
                    n_adopted = adopted
                    assert new_adopt == ref_adopt, f"step {t}: adopted {new_adopt}, oracle {ref_adopt}"
                    assert abs(j - oracle.overlap_ratio(*ref_counts)) <= 0.01, f"step {t}: overlap {j}"
                    decisions.append((t, new_adopt, j))
                    say(f"step {t} probe: overlap {j:.4f} adopted {new_adopt}")
                    if not new_adopt:  # the cached pattern is untouched
                        np.testing.assert_array_equal(now[0], pattern[0])
                        np.testing.assert_array_equal(now[1], pattern[1])
                if act != "PROBE_SPARSE" or decisions[-1][1]:
                    check_topk_rows(csr_rows(*now), A4.reshape(rows, -1), k, f"step {t} pattern")
                pattern = now
            if act == "DENSE" or act == "DENSE_SELECT":
                ro, rl = oracle.dense_attention(hq, hk, hv)
            else:
                ro, rl = oracle.block_sparse_attention(hq, hk, hv, pattern[0], pattern[1], w.block, w.block)
            check_out(to_np(o), ro, to_np(lse), rl, w.dtype, f"step {t} {act}")
        n_probes, adopted, _ = sd.sdattn_schedule_probe_stats(h)
        assert n_probes == acts.count("PROBE_SPARSE") and adopted == sum(d[1] for d in decisions)
    finally:
        sd.sdattn_schedule_destroy(h)
    return decisions


@pytest.mark.parametrize("min_overlap", [0.0, 0.5, 1.0])
def test_tiny_fp32_probe_schedule(min_overlap):
    """Steps 0-3 share a base (fresh Q/V noise only); from step 4 the inputs are
    unrelated ones, so the step-4 probe sees a moved pattern."""
    w = scaled(WORKLOADS["tiny_fp32_h4_l512"], total_steps=8, probe_interval=2, min_overlap=min_overlap)
    say(f"probe schedule tiny fp32 min_overlap={min_overlap}")
    base, other = make_base(w), make_base(scaled(w, wid=101))
    dec = _run_probe_schedule(w, lambda t: make_step(w, t, base if t < 4 else other))
    assert [d[0] for d in dec] == [2, 4, 6]
    assert dec[1][2] < 0.5  # the inputs changed
    if min_overlap == 0.0:
        assert not any(d[1] for d in dec)
    if min_overlap == 0.5:
        assert [d[1] for d in dec] == [False, True, False]


def test_bf16_probe_schedule_128_blocks():
    """bf16, 128-token blocks, a probe at every sparse step: a drifting pattern
    is kept, a replaced one adopted, and the next probes compare against it."""
    w = scaled(WORKLOADS["sparsed_64k"], seq_len=2048, q_heads=4, kv_heads=4, total_steps=7, dense_steps=1,
               select_step=1, keep_frac=0.25, probe_interval=1, min_overlap=0.6)
    say("probe schedule bf16 L=2048 block 128")
    base, other = make_base(w), make_base(scaled(w, wid=102))
    dec = _run_probe_schedule(w, lambda t: make_step(w, t, base if t < 4 else other))
    assert [d[0] for d in dec] == [2, 3, 4, 5, 6]
    assert [d[1] for d in dec] == [False, False, True, False, False]
