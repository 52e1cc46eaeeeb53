"""Helpers of the GPU parity tests: device tensors from the seeded
generator, and the comparison rules (output tolerances and the near-cut
exemption for selected index sets)."""

import numpy as np
import torch

import sparse_bidirectional_attention_amd as sd

# tolerances (bf16 inputs with fp32 accumulation; fp32 path)
BF16_MAX_ABS, BF16_MEAN_ABS = 1e-2, 1e-3
F32_ABS = 1e-5
LSE_BF16, LSE_F32 = 1e-3, 1e-5
SCORE_REL = 1e-5   # debug score outputs (pooled mass, column scores)
CUT_REL = 1e-5     # candidates this close (relative) to a cut are exempt


def say(*a):
    print(*a, flush=True)


def to_dev(x: np.ndarray) -> torch.Tensor:
    """numpy float32 -> float32 device tensor; uint16 bf16 bits -> bf16 device tensor."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def host_inputs(t: torch.Tensor) -> np.ndarray:
    """Exact host copy of a device input (bf16 as uint16 bits, f32 as float32)."""
    if t.dtype == torch.bfloat16:
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def check_out(o_gpu, o_ref, lse_gpu, lse_ref, dtype, what=""):
    o_gpu, o_ref = np.asarray(o_gpu, np.float64), np.asarray(o_ref, np.float64)
    err = np.abs(o_gpu - o_ref)
    if dtype == "bf16":
        assert err.max() <= BF16_MAX_ABS, f"{what}: O max-abs {err.max():.3e}"
        assert err.mean() <= BF16_MEAN_ABS, f"{what}: O mean-abs {err.mean():.3e}"
        ltol = LSE_BF16
    else:
        assert err.max() <= F32_ABS, f"{what}: O max-abs {err.max():.3e}"
        ltol = LSE_F32
    if lse_gpu is not None:
        lse_gpu, lse_ref = np.asarray(lse_gpu, np.float64), np.asarray(lse_ref, np.float64)
        inf_g, inf_r = np.isneginf(lse_gpu), np.isneginf(lse_ref)
        assert np.array_equal(inf_g, inf_r), f"{what}: -inf lse rows differ"
        lerr = np.abs(lse_gpu[~inf_r] - lse_ref[~inf_r])
        if lerr.size:
            assert lerr.max() <= ltol, f"{what}: lse max-abs {lerr.max():.3e}"
    return float(err.max()), float(err.mean())


def check_topk_rows(gpu_sets, scores, k, what=""):
    """Every row keeps exactly k indices; they equal the exact top-k by
    (score desc, index asc) except for candidates within CUT_REL of the cut."""
    n_exempt = 0
    for r, (g, s) in enumerate(zip(gpu_sets, scores)):
        g = np.asarray(g)
        assert len(g) == k, f"{what}: row {r} keeps {len(g)} != {k}"
        assert np.all(np.diff(g) > 0), f"{what}: row {r} not ascending / has duplicates"
        order = np.lexsort((np.arange(len(s)), -s))
        ref = np.sort(order[:k])
        if np.array_equal(g, ref):
            continue
        cut = s[order[k - 1]]
        extra = np.setdiff1d(g, ref)
        missing = np.setdiff1d(ref, g)
        assert np.all(s[extra] >= cut * (1 - CUT_REL)), f"{what}: row {r} keeps {extra} below the cut"
        assert np.all(s[missing] <= cut * (1 + CUT_REL)), f"{what}: row {r} drops {missing} above the cut"
        n_exempt += 1
    return n_exempt


def near_cut_topk(s, k):
    """The exact top-k of one row by (score desc, index asc), and the
    candidates whose score lies within CUT_REL of the row's cut, relative to
    the cut's magnitude (scores may be negative).  Returns (required,
    allowed): the top-k without the near-cut candidates, and the top-k with
    them.  A selection is valid when it holds every required index and only
    allowed ones."""
    s = np.asarray(s, np.float64)
    order = np.lexsort((np.arange(len(s)), -s))
    top = np.sort(order[:k])
    cut = s[order[k - 1]]
    near = np.nonzero(np.abs(s - cut) <= CUT_REL * abs(cut))[0]
    if np.all(np.isin(near, top)):
        return top, top  # no candidate outside the top-k is close to the cut: the set is exact
    return np.setdiff1d(top, near), np.union1d(top, near)


def check_union_of_topk(union, score_rows, k, what=""):
    """A union of per-row top-k selections (the rows of one kv head) against
    the exact per-row selections of the oracle's scores: it must hold every
    index some row requires and only indices some row allows (near-cut
    candidates may go either way).  Returns the number of near-cut indices
    the union holds beyond the rows' exact selections."""
    union = np.asarray(union)
    assert np.all(np.diff(union) > 0), f"{what}: union not ascending / has duplicates"
    required, allowed, exact = [], [], []
    for s in score_rows:
        r, a = near_cut_topk(s, k)
        required.append(r)
        allowed.append(a)
        exact.append(np.lexsort((np.arange(len(s)), -np.asarray(s)))[:k])
    req = np.unique(np.concatenate(required)) if required else np.zeros(0, np.int64)
    alw = np.unique(np.concatenate(allowed)) if allowed else np.zeros(0, np.int64)
    missing = np.setdiff1d(req, union)
    extra = np.setdiff1d(union, alw)
    assert missing.size == 0, f"{what}: union misses required indices {missing[:8]}"
    assert extra.size == 0, f"{what}: union holds indices no row selects {extra[:8]}"
    ex = np.unique(np.concatenate(exact)) if exact else np.zeros(0, np.int64)
    return int(np.setxor1d(union, ex).size)


def check_topk_set(sel, s, k, what=""):
    """One top-k selection (any order, no duplicates, exactly k) against the
    oracle's scores, up to near-cut candidates."""
    sel = np.sort(np.asarray(sel))
    assert len(sel) == k and np.all(np.diff(sel) > 0), f"{what}: {len(sel)} indices, expected {k} distinct"
    req, alw = near_cut_topk(s, k)
    assert np.all(np.isin(req, sel)), f"{what}: misses {np.setdiff1d(req, sel)}"
    assert np.all(np.isin(sel, alw)), f"{what}: holds {np.setdiff1d(sel, alw)}"


def csr_rows(row_ptr, col_idx):
    rp = np.asarray(row_ptr)
    ci = np.asarray(col_idx)
    return [ci[rp[r]:rp[r + 1]] for r in range(len(rp) - 1)]


def dev_csr(row_ptr, col_idx):
    return (torch.from_numpy(np.asarray(row_ptr, np.int32)).cuda(),
            torch.from_numpy(np.asarray(col_idx, np.int32) if len(col_idx) else np.zeros(1, np.int32)).cuda())
