"""The allocation-free pooled selection (sdattn_select_blocks_noalloc)
against the entry point that takes a caller's workspace
(sdattn_select_blocks), through the C ABI.

On the GPU: two calls in a row on the same device, the second with a
smaller problem (so its scratch still holds the first call's contents),
each bit-identical to sdattn_select_blocks on the same inputs (row_ptr,
col_idx and the pooled mass), with both budgets; once the first call on
the device has resolved the scratch, the device's free memory is unchanged
across every later call.  On the host: a selection whose workspace
exceeds the static scratch is refused before anything is enqueued."""

import ctypes

import numpy as np
import pytest
import torch

import sparse_bidirectional_attention_amd as sd
from gpu_util import say, to_dev
from workloads import tiny_random


def _free_bytes():
    free, total = ctypes.c_size_t(0), ctypes.c_size_t(0)
    hip = ctypes.CDLL("libamdhip64.so")
    assert hip.hipMemGetInfo(ctypes.byref(free), ctypes.byref(total)) == 0
    return free.value


def _resolve_scratch():
    """One small call: the first call on a device looks up the scratch's
    device address, and the runtime then holds the array (until the process
    ends); later calls must leave the device's free memory unchanged."""
    x = tiny_random(299, 1, 1, 1, 128, 64, dtype="bf16")
    q, k = to_dev(x["q"]), to_dev(x["k"])
    p = sd.problem_of(q, k)
    budget = sd.topk_budget(0.5)
    _, cap = sd.sdattn_select_blocks_workspace(p, 64, 64, budget)
    rp = torch.empty(3, dtype=torch.int32, device="cuda")
    ci = torch.empty(cap, dtype=torch.int32, device="cuda")
    sd.sdattn_select_blocks_noalloc(p, q, k, 64, 64, budget, rp, ci, cap)
    torch.cuda.synchronize()


def _select_both(seed, B, Hq, Hkv, L, d, block, budget):
    x = tiny_random(seed, B, Hq, Hkv, L, d, dtype="bf16")
    q, k = to_dev(x["q"]), to_dev(x["k"])
    p = sd.problem_of(q, k)
    ws_bytes, cap = sd.sdattn_select_blocks_workspace(p, block, block, budget)
    assert ws_bytes <= sd.NOALLOC_SCRATCH_BYTES
    nqb, nkb = -(-L // block), -(-L // block)
    rows = B * Hq * nqb
    out = {}
    for kind in ("workspace", "noalloc"):
        rp = torch.full((rows + 1,), -7, dtype=torch.int32, device="cuda")
        ci = torch.full((max(cap, 1),), -7, dtype=torch.int32, device="cuda")
        mass = torch.full((rows * nkb,), -1.0, dtype=torch.float32, device="cuda")
        if kind == "workspace":
            ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
            sd.sdattn_select_blocks(p, q, k, block, block, budget, rp, ci, cap, mass, ws, ws_bytes)
        else:
            torch.cuda.synchronize()
            free0 = _free_bytes()
            sd.sdattn_select_blocks_noalloc(p, q, k, block, block, budget, rp, ci, cap, mass)
            torch.cuda.synchronize()
            assert _free_bytes() == free0, "the allocation-free selection changed the device's free memory"
        torch.cuda.synchronize()
        nnz = int(rp[-1].item())
        out[kind] = (rp.cpu().numpy(), ci[:nnz].cpu().numpy(), mass.cpu().numpy())
    for a, b, name in zip(out["workspace"], out["noalloc"], ("row_ptr", "col_idx", "pooled mass")):
        assert np.array_equal(a, b), f"{name} differs"
    return int(out["noalloc"][0][-1]), ws_bytes


@pytest.mark.gpu
@pytest.mark.parametrize("budget_kind", ["topk", "mass"])
def test_noalloc_selection_equals_workspace_selection(budget_kind):
    _resolve_scratch()
    budget = sd.topk_budget(0.1) if budget_kind == "topk" else sd.mass_budget(0.9, 0.15)
    # a first call that fills much of the scratch, then a smaller one on top of its contents
    cases = [(1, 32, 32, 16384, 128, 64), (1, 4, 2, 1000, 64, 128)]
    sizes = []
    for i, (B, Hq, Hkv, L, d, blk) in enumerate(cases):
        say(f"noalloc {budget_kind} call {i}: B{B} Hq{Hq} Hkv{Hkv} L{L} d{d} block {blk}")
        nnz, ws_bytes = _select_both(300 + i, B, Hq, Hkv, L, d, blk, budget)
        sizes.append(ws_bytes)
        say(f"  nnz {nnz}, workspace {ws_bytes} bytes: bit-identical")
    assert sizes[1] < sizes[0]


@pytest.mark.gpu
def test_noalloc_then_workspace_then_noalloc_again():
    """Calls interleaved with the workspace entry point and with each other on
    one stream stay exact (the scratch keeps the last call's contents)."""
    _resolve_scratch()
    for i, (L, blk, budget) in enumerate([(4096, 128, sd.topk_budget(0.05)), (2048, 64, sd.mass_budget(0.95, 0.1)),
                                          (777, 64, sd.topk_budget(0.3))]):
        _select_both(400 + i, 1, 8, 4, L, 128, blk, budget)


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    """64K tokens, 128-token blocks, capped mass: 80 MiB of workspace, more
    than the static scratch; refused on the host (no GPU needed)."""
    p = sd.problem(1, 32, 32, 65536, 128, "bf16")
    budget = sd.mass_budget(0.95, 0.1)
    ws_bytes, cap = sd.sdattn_select_blocks_workspace(p, 128, 128, budget)
    assert ws_bytes > sd.NOALLOC_SCRATCH_BYTES
    bad = ctypes.c_void_p(0x1000)
    st = sd.lib().sdattn_select_blocks_noalloc(ctypes.byref(p), bad, bad, 128, 128, ctypes.byref(budget), bad, bad,
                                               cap, None, None)
    assert st == 5, sd.sdattn_last_error()  # SDATTN_ERR_WORKSPACE
    assert "static scratch" in sd.sdattn_last_error()
