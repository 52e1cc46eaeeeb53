"""The schedule driver on the CPU, against a recording fake backend.

libsdattn_fake.so links the driver and the argument checks (plain C++) with
a backend that logs every call and can fail on purpose; no GPU is used.
The action table is compared with the oracle's, which is written
independently from the same rule.
"""

import ctypes
import os
import random
import re

import pytest

import oracle
import sparse_bidirectional_attention_amd as sd
from sparse_bidirectional_attention_amd import build as sdbuild
from workloads import WORKLOADS
from workloads.configs import scaled

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def fake():
    # SDATTN_FAKE_LIB names another build of the same sources (the sanitized
    # one, tests/test_sanitize_host.py); by default the plain build is used
    path = os.environ.get("SDATTN_FAKE_LIB") or sdbuild.FAKE_LIB
    if path == sdbuild.FAKE_LIB and not os.path.exists(path):
        sdbuild.build_fake()
    lib = sd.declare(ctypes.CDLL(path), required=False)
    lib.sdattn_fake_log_entry.restype = ctypes.c_char_p
    lib.sdattn_fake_log_entry.argtypes = [ctypes.c_int]
    lib.sdattn_fake_reset.argtypes = [ctypes.c_int, ctypes.c_int]
    return lib


def _desc_of(w):
    sel = sd.SEL_KINDS[w.selector]
    budget = sd.topk_budget(w.keep_frac) if w.budget == "topk" else sd.mass_budget(w.mass, w.max_mean_density)
    return sd.schedule_desc(w.total_steps, w.dense_steps, w.select_step, w.refresh_interval, list(w.refresh_steps),
                            w.refresh_dense, sel, w.block, w.block, budget, w.column_keep_frac,
                            w.probe_interval, w.min_overlap)


def _prob_of(w):
    return sd.problem(w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim, w.dtype)


def _create(lib, p, d):
    h = ctypes.c_void_p(None)
    st = lib.sdattn_schedule_create(ctypes.byref(p), ctypes.byref(d), ctypes.byref(h))
    assert st == 0, lib.sdattn_last_error()
    return h


def _actions(lib, h, n):
    out = []
    for t in range(n):
        a = ctypes.c_int(-1)
        assert lib.sdattn_schedule_action(h, t, ctypes.byref(a)) == 0
        out.append(sd.ACTIONS[a.value])
    return out


def _log(lib):
    return [lib.sdattn_fake_log_entry(i).decode() for i in range(lib.sdattn_fake_log_size())]


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_action_table_matches_oracle(fake, name):
    w = WORKLOADS[name]
    h = _create(fake, _prob_of(w), _desc_of(w))
    try:
        ref = oracle.schedule_actions(w.total_steps, w.dense_steps, w.select_step, w.refresh_interval,
                                      w.refresh_steps, w.refresh_dense)
        assert _actions(fake, h, w.total_steps) == ref
    finally:
        fake.sdattn_schedule_destroy(h)
    assert fake.sdattn_fake_live_allocs() == 0


def test_random_schedules_match_oracle(fake):
    rng = random.Random(0)
    p = sd.problem(1, 2, 2, 256, 64, "bf16")
    for _ in range(200):
        T = rng.randint(1, 60)
        dense = rng.randint(0, T)
        sel = rng.randint(0, min(dense, T - 1))
        interval = rng.choice([0, 0, 1, 3, 7])
        refresh = tuple(sorted(rng.sample(range(T), rng.randint(0, min(4, T)))))
        rdense = rng.random() < 0.5
        probe = rng.choice([0, 0, 1, 2, 5])
        d = sd.schedule_desc(T, dense, sel, interval, list(refresh), rdense, budget=sd.topk_budget(0.5),
                             probe_interval=probe, min_overlap=0.5)
        h = _create(fake, p, d)
        ref = oracle.schedule_actions(T, dense, sel, interval, refresh, rdense, probe)
        assert _actions(fake, h, T) == ref
        fake.sdattn_schedule_destroy(h)
    assert fake.sdattn_fake_live_allocs() == 0


def test_split_rows_schedule_runs_every_sparse_step_over_the_split_plan(fake):
    """With split_rows, every selection is followed by the split plan of its
    row_ptr, into that buffer's workspace, and every sparse step runs the
    split forward over the most recent one; the dispatch-plan calls are not
    made.  split_rows must be 0 or 1, and is refused for column patterns."""
    w = WORKLOADS["llada8b_8k"]
    d = _desc_of(w)
    d.split_rows = 1
    h = _create(fake, _prob_of(w), d)
    fake.sdattn_fake_reset(-1, 0)
    try:
        for t in range(w.total_steps):
            assert _step(fake, h, t) == 0
        log = _log(fake)
        assert not any(l.startswith(("block_plan", "block_sparse ")) for l in log)
        cur = ws = None
        n_sparse, wss = 0, []
        for i, l in enumerate(log):
            if l.startswith("select_blocks"):
                cur = re.search(r"rp=(\S+) ci=(\S+)", l).groups()
                nxt = log[i + 1]
                assert nxt.startswith("block_split_plan") and re.search(r"rp=(\S+)", nxt).group(1) == cur[0]
                assert "bytes=1048576" in nxt and "bq=64 bk=64" in nxt
                ws = re.search(r"ws=(\S+)", nxt).group(1)
                wss.append(ws)
            elif l.startswith("block_sparse_split"):
                assert re.search(r"rp=(\S+) ci=(\S+)", l).groups() == cur
                assert re.search(r"ws=(\S+)", l).group(1) == ws and "bytes=1048576" in l
                n_sparse += 1
        assert n_sparse == 255 and wss[0] != wss[1] and wss[0] == wss[2]
    finally:
        fake.sdattn_schedule_destroy(h)
    assert fake.sdattn_fake_live_allocs() == 0
    for bad, code in ((2, 2), (-1, 2)):
        d.split_rows = bad
        hh = ctypes.c_void_p(None)
        assert fake.sdattn_schedule_create(ctypes.byref(_prob_of(w)), ctypes.byref(d), ctypes.byref(hh)) == code
    wc = WORKLOADS["pulsecol_dream7b_16k"]
    dc = _desc_of(wc)
    dc.split_rows = 1
    hh = ctypes.c_void_p(None)
    assert fake.sdattn_schedule_create(ctypes.byref(_prob_of(wc)), ctypes.byref(dc), ctypes.byref(hh)) == 8
    assert fake.sdattn_fake_live_allocs() == 0


def _step(lib, h, t, o=0x5000, lse=None):
    return lib.sdattn_schedule_step(h, t, ctypes.c_void_p(0x1000), ctypes.c_void_p(0x2000),
                                    ctypes.c_void_p(0x3000), ctypes.c_void_p(o), lse, None)


def test_block_schedule_reuses_and_refreshes(fake):
    w = WORKLOADS["llada8b_8k"]
    h = _create(fake, _prob_of(w), _desc_of(w))
    fake.sdattn_fake_reset(-1, 0)
    for t in range(w.total_steps):
        assert _step(fake, h, t) == 0
    log = _log(fake)
    sel = [l for l in log if l.startswith("select_blocks")]
    sparse = [l for l in log if l.startswith("block_sparse")]
    assert len(sel) == 8 and len(sparse) == 255 and log[0].startswith("dense")
    assert all("cap=52428" in l for l in sel)
    # every selection is followed by the dispatch plan of its row_ptr; every
    # sparse step uses the CSR and the plan of the most recent selection;
    # buffers alternate
    cur = plan = None
    bufs, plans = [], []
    for i, l in enumerate(log):
        if l.startswith("select_blocks"):
            cur = re.search(r"rp=(\S+) ci=(\S+)", l).groups()
            bufs.append(cur)
            assert log[i + 1].startswith("block_plan") and re.search(r"rp=(\S+)", log[i + 1]).group(1) == cur[0]
            assert "bq=64 bk=64" in log[i + 1]
            plan = re.search(r"plan=(\S+)", log[i + 1]).group(1)
            plans.append(plan)
        elif l.startswith("block_sparse"):
            assert re.search(r"rp=(\S+) ci=(\S+)", l).groups() == cur
            assert re.search(r"plan=(\S+)", l).group(1) == plan
    assert bufs[0] != bufs[1] and bufs[0] == bufs[2]
    assert plans[0] != plans[1] and plans[0] == plans[2] and "(nil)" not in plans
    counts = (ctypes.c_int64 * 4)()
    last = ctypes.c_int32(0)
    assert fake.sdattn_schedule_stats(h, counts, ctypes.byref(last)) == 0
    assert list(counts) == [0, 1, 7, 248] and last.value == 224
    fake.sdattn_schedule_destroy(h)


def test_failed_selection_keeps_the_cached_pattern(fake):
    w = WORKLOADS["llada8b_8k"]
    h = _create(fake, _prob_of(w), _desc_of(w))
    fake.sdattn_fake_reset(-1, 0)
    assert _step(fake, h, 0) == 0
    rp, ci, cap = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_int64()
    assert fake.sdattn_schedule_mask(h, ctypes.byref(rp), ctypes.byref(ci), ctypes.byref(cap)) == 0
    before = (rp.value, ci.value)
    fake.sdattn_fake_reset(0, 7)  # the next backend call (the step-32 selection) fails
    assert _step(fake, h, 32) == 7
    assert "injected" in fake.sdattn_last_error().decode()
    assert fake.sdattn_schedule_mask(h, ctypes.byref(rp), ctypes.byref(ci), ctypes.byref(cap)) == 0
    assert (rp.value, ci.value) == before
    fake.sdattn_fake_reset(1, 7)  # the selection succeeds, its dispatch plan fails: still the cached pattern
    assert _step(fake, h, 32) == 7
    assert [l.split()[0] for l in _log(fake)] == ["select_blocks", "FAIL"]
    assert fake.sdattn_schedule_mask(h, ctypes.byref(rp), ctypes.byref(ci), ctypes.byref(cap)) == 0
    assert (rp.value, ci.value) == before
    fake.sdattn_fake_reset(-1, 0)
    assert _step(fake, h, 33) == 0
    assert re.search(r"rp=(\S+)", _log(fake)[0]).group(1) == hex(before[0])
    counts = (ctypes.c_int64 * 4)()
    last = ctypes.c_int32(0)
    fake.sdattn_schedule_stats(h, counts, ctypes.byref(last))
    assert list(counts) == [0, 1, 0, 1] and last.value == 0
    fake.sdattn_schedule_destroy(h)


def test_sparse_step_before_any_pattern_is_a_state_error(fake):
    w = WORKLOADS["sparsed_64k"]
    h = _create(fake, _prob_of(w), _desc_of(w))
    fake.sdattn_fake_reset(-1, 0)
    assert _step(fake, h, 500) == 9
    assert _log(fake) == []
    rp, ci, cap = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_int64()
    assert fake.sdattn_schedule_mask(h, ctypes.byref(rp), ctypes.byref(ci), ctypes.byref(cap)) == 9
    assert _step(fake, h, 10) == 0 and _log(fake)[0].startswith("dense")
    assert _step(fake, h, 205) == 0
    assert _step(fake, h, 500) == 0
    assert _step(fake, h, 1024) == 2 and _step(fake, h, -1) == 2
    fake.sdattn_schedule_destroy(h)


def test_column_schedule_uses_own_lse_buffer(fake):
    w = WORKLOADS["pulsecol_dream7b_16k"]
    h = _create(fake, _prob_of(w), _desc_of(w))
    fake.sdattn_fake_reset(-1, 0)
    for t in range(w.total_steps):
        assert _step(fake, h, t) == 0
    log = _log(fake)
    dense = [l for l in log if l.startswith("dense")]
    sel = [l for l in log if l.startswith("select_columns")]
    assert len(dense) == 3 and len(sel) == 3 and all("kcol=492" in l for l in sel)
    for d, s in zip(dense, sel):  # dense writes the lse that the selection reads
        assert re.search(r"lse=(\S+)", d).group(1) == re.search(r"lse=(\S+)", s).group(1) != "(nil)"
    # sparse steps: the kept rows gathered into the handle's buffers, then the packed forward
    gathers = [l for l in log if l.startswith("gather_columns")]
    packed = [l for l in log if l.startswith("column_packed")]
    assert len(gathers) == len(packed) == 189 and not any(l.startswith("column_sparse") for l in log)
    kc, vc = re.search(r"kc=(\S+) vc=(\S+)", gathers[0]).groups()
    assert all(f"kc={kc} vc={vc}" in l for l in gathers + packed) and "kcol=492" in packed[0]
    cur = None
    for l in log:  # every gather reads the most recent selection's columns
        if l.startswith("select_columns"):
            cur = re.search(r"ci=(\S+)", l).group(1)
        elif l.startswith("gather_columns"):
            assert re.search(r"ci=(\S+)", l).group(1) == cur
    fake.sdattn_schedule_destroy(h)
    assert fake.sdattn_fake_live_allocs() == 0


def _probe_desc(**kw):
    w = scaled(WORKLOADS["llada8b_8k"], total_steps=12, refresh_interval=8, probe_interval=3, min_overlap=0.7)
    return w, _desc_of(scaled(w, **kw))


def test_probe_step_selects_into_the_idle_buffer_and_adopts_over_the_cached_one(fake):
    w, d = _probe_desc()
    fake.sdattn_fake_reset(-1, 0)
    h = _create(fake, _prob_of(w), d)
    init = _log(fake)
    assert len(init) == 1 and init[0].startswith("probe_init")
    state = re.search(r"state=(\S+)", init[0]).group(1)
    assert _actions(fake, h, 12) == oracle.schedule_actions(12, 1, 0, 8, (), False, 3)
    fake.sdattn_fake_reset(-1, 0)
    for t in range(12):
        assert _step(fake, h, t) == 0
    log = _log(fake)
    cached = re.search(r"rp=(\S+) ci=(\S+)", [l for l in log if l.startswith("select_blocks")][0]).groups()
    i = 0
    probes = 0
    while i < len(log):
        l = log[i]
        if l.startswith("select_blocks") and i + 1 < len(log) and log[i + 1].startswith("overlap"):
            # a probe: selection into the idle buffer, overlap(cached, probe),
            # adoption of the probe over the cached buffer, the cached buffer's
            # dispatch plan computed again, attention on the cached buffer
            probe_buf = re.search(r"rp=(\S+) ci=(\S+)", l).groups()
            assert probe_buf != cached
            ov, ad, pl, bs = log[i + 1], log[i + 2], log[i + 3], log[i + 4]
            assert pl.startswith("block_plan") and re.search(r"rp=(\S+)", pl).group(1) == cached[0]
            assert re.search(r"plan=(\S+)", bs).group(1) == re.search(r"plan=(\S+)", pl).group(1)
            assert re.search(r"a=(\S+),(\S+) b=(\S+),(\S+)", ov).groups() == cached + probe_buf
            assert f"rows={32 * 128}" in ov
            assert re.search(r"dst=(\S+),(\S+) src=(\S+),(\S+)", ad).groups() == cached + probe_buf
            assert re.search(r"counts=(\S+)", ad).group(1) == re.search(r"counts=(\S+)", ov).group(1)
            assert f"state={state}" in ad and "min_overlap=0.7" in ad and "max_copy=52428" in ad
            assert bs.startswith("block_sparse") and re.search(r"rp=(\S+) ci=(\S+)", bs).groups() == cached
            probes += 1
            i += 5
            continue
        if l.startswith("select_blocks"):  # a scheduled refresh switches buffers
            cached = re.search(r"rp=(\S+) ci=(\S+)", l).groups()
        i += 1
    assert probes == 3  # steps 3, 6 and 9; the refresh at step 8 switches buffers before the last one
    n, a, j = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_double()
    assert fake.sdattn_schedule_probe_stats(h, ctypes.byref(n), ctypes.byref(a), ctypes.byref(j), None) == 0
    assert (n.value, a.value) == (probes, 0)
    fake.sdattn_schedule_destroy(h)
    assert fake.sdattn_fake_live_allocs() == 0


def test_probe_descriptor_checks(fake):
    w = WORKLOADS["llada8b_8k"]
    p = _prob_of(w)
    cases = [
        (_desc_of(scaled(w, probe_interval=-1)), 2),
        (_desc_of(scaled(w, probe_interval=4, min_overlap=1.5)), 4),
        (_desc_of(scaled(w, probe_interval=4, min_overlap=-0.1)), 4),
        (_desc_of(scaled(WORKLOADS["pulsecol_dream7b_16k"], probe_interval=4, min_overlap=0.5)), 8),
    ]
    for d, want in cases:
        h = ctypes.c_void_p(None)
        assert fake.sdattn_schedule_create(ctypes.byref(p), ctypes.byref(d), ctypes.byref(h)) == want
        assert h.value is None
    # min_overlap is not checked when there are no probes; 0 and 1 are valid thresholds
    for d in (_desc_of(scaled(w, min_overlap=7.0)), _desc_of(scaled(w, probe_interval=2, min_overlap=0.0)),
              _desc_of(scaled(w, probe_interval=2, min_overlap=1.0))):
        h = _create(fake, p, d)
        fake.sdattn_schedule_destroy(h)
    assert fake.sdattn_fake_live_allocs() == 0


def test_probe_step_errors_leave_the_pattern_alone(fake):
    w, d = _probe_desc()
    h = _create(fake, _prob_of(w), d)
    fake.sdattn_fake_reset(-1, 0)
    assert _step(fake, h, 3) == 9 and _log(fake) == []  # no pattern yet
    assert _step(fake, h, 0) == 0
    fake.sdattn_fake_reset(-1, 0)
    assert _step(fake, h, 3, o=0) == 1 and _log(fake) == []  # NULL output: nothing enqueued
    fake.sdattn_fake_reset(0, 7)  # the probe's selection fails: no overlap, no adoption
    assert _step(fake, h, 3) == 7
    assert len(_log(fake)) == 1 and _log(fake)[0].startswith("FAIL select_blocks")
    fake.sdattn_fake_reset(1, 7)  # the overlap fails: no adoption, no attention
    assert _step(fake, h, 3) == 7
    assert [l.split()[0] for l in _log(fake)] == ["select_blocks", "FAIL"]
    n, a, j = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_double()
    assert fake.sdattn_schedule_probe_stats(h, ctypes.byref(n), ctypes.byref(a), ctypes.byref(j), None) == 0
    assert (n.value, a.value, j.value) == (0, 0, 1.0)
    fake.sdattn_fake_reset(-1, 0)
    assert _step(fake, h, 3) == 0
    assert [l.split()[0] for l in _log(fake)] == ["select_blocks", "overlap", "probe_adopt", "block_plan",
                                                  "block_sparse"]
    fake.sdattn_schedule_destroy(h)
    assert fake.sdattn_fake_live_allocs() == 0


def test_exact_selector_schedule_uses_the_dense_lse(fake):
    w = scaled(WORKLOADS["sparsed_64k"], selector="blocks_exact", refresh_dense=True, total_steps=10, dense_steps=4,
               select_step=3, refresh_interval=4)
    d = _desc_of(w)
    assert d.sel == sd.SDATTN_SEL_BLOCKS_EXACT
    h = _create(fake, _prob_of(w), d)
    assert _actions(fake, h, 10) == ["DENSE", "DENSE", "DENSE", "DENSE_SELECT", "SPARSE", "SPARSE", "SPARSE",
                                     "DENSE_SELECT", "SPARSE", "SPARSE"]
    fake.sdattn_fake_reset(-1, 0)
    for t in range(10):
        assert _step(fake, h, t) == 0  # lse = NULL: the handle's own buffer
    log = _log(fake)
    sel = [i for i, l in enumerate(log) if l.startswith("select_blocks_exact")]
    assert len(sel) == 2 and not any(l.startswith("select_blocks ") for l in log)
    for i in sel:  # the dense pass right before writes the lse the selection reads
        assert log[i - 1].startswith("dense")
        own = re.search(r"lse=(\S+)", log[i - 1]).group(1)
        assert own != "(nil)" and re.search(r"lse=(\S+)", log[i]).group(1) == own
        assert "cap=425984" in log[i]
    # sparse steps use the pattern of the latest selection (applies from the
    # next step) and the dispatch plan computed right after it
    cur = plan = None
    for i, l in enumerate(log):
        if l.startswith("select_blocks_exact"):
            cur = re.search(r"rp=(\S+) ci=(\S+)", l).groups()
            assert log[i + 1].startswith("block_plan") and re.search(r"rp=(\S+)", log[i + 1]).group(1) == cur[0]
            plan = re.search(r"plan=(\S+)", log[i + 1]).group(1)
        elif l.startswith("block_sparse"):
            assert re.search(r"rp=(\S+) ci=(\S+)", l).groups() == cur
            assert re.search(r"plan=(\S+)", l).group(1) == plan
    # a caller lse is used when given
    fake.sdattn_fake_reset(-1, 0)
    assert _step(fake, h, 3, lse=ctypes.c_void_p(0x7000)) == 0
    assert all("lse=0x7000" in l for l in _log(fake)[:2])
    fake.sdattn_schedule_destroy(h)
    assert fake.sdattn_fake_live_allocs() == 0


def test_exact_selector_descriptor_checks(fake):
    w = scaled(WORKLOADS["sparsed_64k"], selector="blocks_exact", total_steps=10, dense_steps=4, select_step=3,
               refresh_dense=True)
    p = _prob_of(w)
    for kw, want in [(dict(refresh_dense=False), 2), (dict(select_step=4), 2),
                     (dict(probe_interval=2, min_overlap=0.5), 8)]:
        d = _desc_of(scaled(w, **kw))
        h = ctypes.c_void_p(None)
        assert fake.sdattn_schedule_create(ctypes.byref(p), ctypes.byref(d), ctypes.byref(h)) == want
    assert fake.sdattn_fake_live_allocs() == 0
