"""GPU parity of the exact block-mass selector against the fp64 oracle.

The mass of every (query block, key block) pair is compared with the oracle's
exact block mass (1e-5 relative); the selected index sets must match the
oracle's selection from its own exact mass except for candidates within 1e-5
(relative) of a row's cut.  The lse the GPU selector reads comes from the
library's own dense forward, as in a schedule; the oracle uses its own fp64
lse.  Schedules with the exact selector run through the C-ABI driver.
"""

import numpy as np
import pytest
import torch

import oracle
import sparse_bidirectional_attention_amd as sd
from gpu_util import SCORE_REL, check_out, check_topk_rows, csr_rows, host_inputs, say, to_dev, to_np
from test_gpu_probe import _d2h
from test_gpu_select import _check_mass_rows
from workloads import WORKLOADS, make_base, make_step, tiny_random
from workloads.configs import scaled

pytestmark = pytest.mark.gpu

MASS_ABS = 1e-12  # absolute floor for the mass comparison (sums of fp32 exponentials)


def _dev(x):
    return {n: to_dev(a) for n, a in x.items()}


def _dense_lse(x):
    p = sd.problem_of(x["q"], x["k"])
    o = torch.empty_like(x["q"])
    lse = torch.empty(x["q"].shape[:3], dtype=torch.float32, device="cuda")
    sd.sdattn_forward_dense(p, x["q"], x["k"], x["v"], o, lse)
    return lse


def _select_exact(x, lse, bq, bk, budget):
    p = sd.problem_of(x["q"], x["k"])
    ws_bytes, nnz = sd.sdattn_select_blocks_exact_workspace(p, bq, bk, budget)
    L = x["q"].shape[2]
    rows = x["q"].shape[0] * x["q"].shape[1] * (-(-L // bq))
    nkb = -(-L // bk)
    rp = torch.empty(rows + 1, dtype=torch.int32, device="cuda")
    ci = torch.full((max(nnz, 1),), -1, dtype=torch.int32, device="cuda")
    mass = torch.empty(rows * nkb, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    sd.sdattn_select_blocks_exact(p, x["q"], x["k"], lse, bq, bk, budget, rp, ci, nnz, mass, ws, ws_bytes)
    torch.cuda.synchronize()
    return rp.cpu().numpy(), ci.cpu().numpy(), mass.cpu().numpy().astype(np.float64).reshape(rows, nkb)


def _oracle_mass(x, bq, bk):
    hq, hk, hv = (host_inputs(x[n]) for n in "qkv")
    _, rl = oracle.dense_attention(hq, hk, hv)
    return oracle.exact_block_mass(hq, hk, rl, bq, bk)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("Hq,Hkv,L,d,bq,bk,frac", [(4, 2, 1000, 128, 64, 64, 0.25), (4, 4, 1300, 128, 128, 128, 0.1),
                                                   (6, 2, 777, 64, 64, 128, 0.3), (2, 1, 700, 128, 128, 64, 0.3),
                                                   (2, 2, 65, 64, 64, 64, 0.5), (3, 3, 4096, 128, 128, 128, 0.05)])
def test_exact_mass_and_topk_match_oracle(dtype, Hq, Hkv, L, d, bq, bk, frac):
    say(f"select_blocks_exact topk {dtype} Hq={Hq} Hkv={Hkv} L={L} d={d} bq={bq} bk={bk} frac={frac}")
    x = _dev(tiny_random(3 * L + Hq, 1, Hq, Hkv, L, d, dtype, scale=1.0))
    lse = _dense_lse(x)
    rp, ci, mass = _select_exact(x, lse, bq, bk, sd.topk_budget(frac))
    A4 = _oracle_mass(x, bq, bk)
    A = A4.reshape(-1, A4.shape[-1])
    np.testing.assert_allclose(mass, A, rtol=SCORE_REL, atol=MASS_ABS)
    np.testing.assert_allclose(mass.sum(-1), 1.0, rtol=1e-5)
    k = oracle.count_from_fraction(frac, A.shape[1])
    assert rp[0] == 0 and np.all(np.diff(rp) == k)
    n_ex = check_topk_rows(csr_rows(rp, ci), A, k, "exact topk")
    say(f"  rows with exempt near-cut differences: {n_ex} of {len(A)}")


@pytest.mark.parametrize("mass,cap,L,bq", [(0.95, 0.10, 4096, 64), (0.5, 0.3, 3000, 128), (0.95, 0.02, 2048, 64)])
def test_exact_mass_cap_selection_matches_oracle(mass, cap, L, bq):
    w = scaled(WORKLOADS["llada8b_8k"], seq_len=L, q_heads=8, kv_heads=8, block=bq)
    say(f"select_blocks_exact mass={mass} cap={cap} L={L} bq={bq}")
    x = _dev(make_step(w, 0))
    lse = _dense_lse(x)
    rp, ci, gmass = _select_exact(x, lse, bq, bq, sd.mass_budget(mass, cap))
    A4 = _oracle_mass(x, bq, bq)
    A = A4.reshape(-1, A4.shape[-1])
    np.testing.assert_allclose(gmass, A, rtol=SCORE_REL, atol=MASS_ABS)
    rrp, rci, tau = oracle.select_mass_cap(A4, mass, cap)
    say(f"  oracle tau*={tau:.6f} nnz={rrp[-1]} gpu nnz={rp[-1]} density={rp[-1] / A.size:.4f}")
    _check_mass_rows(rp, ci, A, tau, mass, cap)


def test_exact_mass_sampled_at_the_64k_shape():
    """The 64K configuration's shape and budget (32 heads, 128-token blocks,
    top 5%): the full selection on the GPU after its dense forward; the oracle
    computes eight sampled query blocks (first and last included), each
    against all 65,536 keys of its head."""
    w = WORKLOADS["sparsed_64k"]
    L, H, bq = w.seq_len, w.q_heads, w.block
    say("select_blocks_exact sampled 64K")
    g = torch.Generator(device="cuda").manual_seed(64)
    x = {n: torch.randn(1, H, L, 128, device="cuda", dtype=torch.float32, generator=g).to(torch.bfloat16)
         for n in "qkv"}
    lse = _dense_lse(x)
    rp, ci, mass = _select_exact(x, lse, bq, bq, sd.topk_budget(w.keep_frac))
    nqb = L // bq
    k = oracle.count_from_fraction(w.keep_frac, nqb)
    assert np.all(np.diff(rp) == k)
    rng = np.random.default_rng(0)
    picks = [(0, 0), (H - 1, nqb - 1)] + [(int(rng.integers(H)), int(rng.integers(nqb))) for _ in range(6)]
    for h, I in picks:
        rows = slice(I * bq, (I + 1) * bq)
        hq = host_inputs(x["q"][:, h:h + 1, rows].contiguous())
        hk = host_inputs(x["k"][:, h:h + 1].contiguous())
        hv = host_inputs(x["v"][:, h:h + 1].contiguous())
        _, rl = oracle.dense_attention(hq, hk, hv)  # these query rows against all keys
        a = oracle.exact_block_mass(hq, hk, rl, bq, bq)[0, 0, 0]
        r = h * nqb + I
        np.testing.assert_allclose(mass[r], a, rtol=SCORE_REL, atol=MASS_ABS)
        check_topk_rows([ci[rp[r]:rp[r + 1]]], a[None], k, f"64K exact row h={h} I={I}")


def test_exact_mass_at_the_largest_key_block_count():
    """L = 65,536 with 64-token blocks: 1,024 key blocks per row, the selector's
    largest row (two heads; sampled rows checked against the oracle)."""
    L, H, bq = 65536, 2, 64
    say("select_blocks_exact nKB=1024")
    g = torch.Generator(device="cuda").manual_seed(1024)
    x = {n: torch.randn(1, H, L, 128, device="cuda", dtype=torch.float32, generator=g).to(torch.bfloat16)
         for n in "qkv"}
    lse = _dense_lse(x)
    rp, ci, mass = _select_exact(x, lse, bq, bq, sd.topk_budget(0.05))
    nqb = L // bq
    k = oracle.count_from_fraction(0.05, nqb)
    assert k == 52 and np.all(np.diff(rp) == k)
    for h, I in [(0, 0), (1, nqb - 1), (0, 517), (1, 3)]:
        rows = slice(I * bq, (I + 1) * bq)
        hq = host_inputs(x["q"][:, h:h + 1, rows].contiguous())
        hk = host_inputs(x["k"][:, h:h + 1].contiguous())
        _, rl = oracle.dense_attention(hq, hk, host_inputs(x["v"][:, h:h + 1].contiguous()))
        a = oracle.exact_block_mass(hq, hk, rl, bq, bq)[0, 0, 0]
        r = h * nqb + I
        np.testing.assert_allclose(mass[r], a, rtol=SCORE_REL, atol=MASS_ABS)
        check_topk_rows([ci[rp[r]:rp[r + 1]]], a[None], k, f"nKB=1024 exact row h={h} I={I}")


def test_exact_selector_schedule_bf16():
    """Through the driver: warm-up, the exact selection on the last dense
    step (pattern from the next step on), a dense refresh, sparse steps."""
    w = scaled(WORKLOADS["sparsed_64k"], seq_len=2048, q_heads=4, kv_heads=4, total_steps=7, dense_steps=3,
               select_step=2, refresh_interval=3, refresh_dense=True, selector="blocks_exact", keep_frac=0.25)
    say("schedule exact selector bf16 L=2048 T=7")
    base = make_base(w)
    acts = oracle.schedule_actions(w.total_steps, w.dense_steps, w.select_step, w.refresh_interval,
                                   w.refresh_steps, w.refresh_dense)
    assert acts == ["DENSE", "DENSE", "DENSE_SELECT", "SPARSE", "SPARSE", "DENSE_SELECT", "SPARSE"]
    p = sd.problem(w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.dtype)
    d = sd.schedule_desc(w.total_steps, w.dense_steps, w.select_step, w.refresh_interval, [], True,
                         sd.SDATTN_SEL_BLOCKS_EXACT, w.block, w.block, sd.topk_budget(w.keep_frac))
    h = sd.sdattn_schedule_create(p, d)
    rows = w.q_heads * (w.seq_len // w.block)
    k = oracle.count_from_fraction(w.keep_frac, w.seq_len // w.block)
    pattern = None
    try:
        for t in range(w.total_steps):
            x = _dev(make_step(w, t, base))
            o = torch.empty_like(x["q"])
            lse = torch.empty(x["q"].shape[:3], dtype=torch.float32, device="cuda")
            assert sd.sdattn_schedule_action(h, t) == acts[t]
            sd.sdattn_schedule_step(h, t, x["q"], x["k"], x["v"], o, None if t == 2 else lse)
            torch.cuda.synchronize()
            hq, hk, hv = (host_inputs(x[n]) for n in "qkv")
            if acts[t] == "SPARSE":
                ro, rl = oracle.block_sparse_attention(hq, hk, hv, pattern[0], pattern[1], w.block, w.block)
            else:
                ro, rl = oracle.dense_attention(hq, hk, hv)
            check_out(to_np(o), ro, None if t == 2 else to_np(lse), rl, "bf16", f"step {t} {acts[t]}")
            if acts[t] == "DENSE_SELECT":
                rp_ptr, ci_ptr, _ = sd.sdattn_schedule_mask(h)
                rpn = _d2h(rp_ptr, rows + 1)
                cin = _d2h(ci_ptr, int(rpn[-1]))
                A = oracle.exact_block_mass(hq, hk, rl, w.block, w.block).reshape(rows, -1)
                check_topk_rows(csr_rows(rpn, cin), A, k, f"step {t} exact pattern")
                pattern = (rpn, cin)
        stats, last = sd.sdattn_schedule_stats(h)
        assert stats["DENSE_SELECT"] == 2 and last == 5
    finally:
        sd.sdattn_schedule_destroy(h)
