"""The C ABI on the CPU: the library loads, exports every declared entry
point, and rejects invalid arguments on the host before touching a GPU."""

import ctypes
import os
import re
import subprocess

import pytest

import sparse_bidirectional_attention_amd as sd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdattn.h")

BAD = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails validation first


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SDATTN_API\s+[\w\s\*]*?\b(sdattn_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) == 32
    out = subprocess.run(["nm", "-D", "--defined-only", sd.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(sdattn_\w+)", out))
    assert set(names) == exported  # nothing missing, nothing extra
    lib = ctypes.CDLL(sd.LIB_PATH)
    for n in names:
        assert getattr(lib, n) is not None
    assert set(names) == set(sd._SIGS)  # the binding declares all of them


def test_version_and_status_strings():
    assert sd.sdattn_abi_version() == sd.SDATTN_ABI_VERSION == 6
    hdr = open(os.path.join(ROOT, "include", "sdattn.h")).read()
    assert f"#define SDATTN_ABI_VERSION {sd.SDATTN_ABI_VERSION}" in hdr
    for i, name in enumerate(sd.STATUS_NAMES):
        assert sd.sdattn_status_string(i) == name


def _st(fn, *args):
    return getattr(sd.lib(), fn)(*args)


def test_problem_validation():
    lib = sd.lib()
    assert lib.sdattn_forward_dense(None, BAD, BAD, BAD, BAD, None, None) == 1  # NULL problem
    cases = [
        (sd.problem(1, 4, 3, 64, 64, "f32"), 2),    # Hq % Hkv
        (sd.problem(0, 4, 4, 64, 64, "f32"), 2),    # batch
        (sd.problem(1, 4, 4, -1, 64, "f32"), 2),    # seq_len
        (sd.problem(1, 4, 4, 64, 96, "f32"), 8),    # head_dim unsupported
        (sd.Problem(1, 4, 4, 64, 64, 7, 0.0), 3),   # dtype
        (sd.problem(1, 4, 4, 64, 64, "f32", float("nan")), 2),
    ]
    for p, code in cases:
        assert lib.sdattn_forward_dense(ctypes.byref(p), BAD, BAD, BAD, BAD, None, None) == code, sd.sdattn_last_error()
    p = sd.problem(1, 4, 4, 64, 64, "bf16")
    assert lib.sdattn_forward_dense(ctypes.byref(p), None, BAD, BAD, BAD, None, None) == 1
    assert "non-NULL" in sd.sdattn_last_error()
    # L == 0 is a no-op that succeeds without touching memory
    p0 = sd.problem(1, 4, 4, 0, 64, "bf16")
    assert lib.sdattn_forward_dense(ctypes.byref(p0), None, None, None, None, None, None) == 0


def test_block_select_validation_and_workspace():
    p = sd.problem(1, 32, 32, 65536, 128, "bf16")
    ws, nnz = sd.sdattn_select_blocks_workspace(p, 128, 128, sd.topk_budget(0.05))
    assert nnz == 32 * 512 * 26 and ws > 0
    p8 = sd.problem(1, 32, 32, 8192, 128, "bf16")
    ws, nnz = sd.sdattn_select_blocks_workspace(p8, 64, 64, sd.mass_budget(0.95, 0.10))
    assert nnz == 52428
    p3 = sd.problem(1, 32, 32, 32768, 128, "bf16")
    assert sd.sdattn_select_blocks_workspace(p3, 128, 128, sd.topk_budget(0.10))[1] == 32 * 256 * 26
    lib = sd.lib()
    with pytest.raises(sd.SdattnError, match="BUDGET"):
        sd.sdattn_select_blocks_workspace(p, 128, 128, sd.topk_budget(0.0))
    with pytest.raises(sd.SdattnError, match="BUDGET"):
        sd.sdattn_select_blocks_workspace(p, 128, 128, sd.mass_budget(1.5))
    with pytest.raises(sd.SdattnError, match="UNSUPPORTED"):
        sd.sdattn_select_blocks_workspace(p, 32, 128, sd.topk_budget(0.1))
    with pytest.raises(sd.SdattnError, match="UNSUPPORTED"):  # nKB = 2048 > 1024
        sd.sdattn_select_blocks_workspace(sd.problem(1, 1, 1, 131072, 128, "bf16"), 64, 64, sd.topk_budget(0.1))
    b = sd.topk_budget(0.05)
    ws, nnz = sd.sdattn_select_blocks_workspace(p, 128, 128, b)
    r = lib.sdattn_select_blocks(ctypes.byref(p), BAD, BAD, 128, 128, ctypes.byref(b), BAD, BAD, nnz - 1, None,
                                 BAD, ws, None)
    assert r == 6 and "col_capacity" in sd.sdattn_last_error()
    r = lib.sdattn_select_blocks(ctypes.byref(p), BAD, BAD, 128, 128, ctypes.byref(b), BAD, BAD, nnz, None,
                                 BAD, ws - 1, None)
    assert r == 5
    r = lib.sdattn_select_blocks(ctypes.byref(p), BAD, BAD, 128, 128, ctypes.byref(b), None, BAD, nnz, None,
                                 BAD, ws, None)
    assert r == 1


def test_sparse_and_column_validation():
    lib = sd.lib()
    p = sd.problem(1, 28, 4, 16384, 128, "bf16")
    assert lib.sdattn_forward_block_sparse(ctypes.byref(p), BAD, BAD, BAD, 96, 128, BAD, BAD, BAD, None, None) == 8
    assert lib.sdattn_forward_block_sparse(ctypes.byref(p), BAD, BAD, BAD, 64, 64, None, BAD, BAD, None, None) == 1
    # dispatch plan: block sizes, NULL row_ptr / plan, L == 0 a no-op; the planned forward checks as the plain one
    assert lib.sdattn_block_plan(ctypes.byref(p), 96, 128, BAD, BAD, None) == 8
    assert lib.sdattn_block_plan(ctypes.byref(p), 64, 64, None, BAD, None) == 1
    assert lib.sdattn_block_plan(ctypes.byref(p), 64, 64, BAD, None, None) == 1
    p0 = sd.problem(1, 28, 4, 0, 128, "bf16")
    assert lib.sdattn_block_plan(ctypes.byref(p0), 64, 64, None, None, None) == 0
    assert lib.sdattn_forward_block_sparse_planned(ctypes.byref(p), BAD, BAD, BAD, 96, 128, BAD, BAD, BAD, BAD, None,
                                                   None) == 8
    assert lib.sdattn_forward_block_sparse_planned(ctypes.byref(p), BAD, BAD, BAD, 64, 64, BAD, None, BAD, BAD, None,
                                                   None) == 1
    # split plan: block sizes, NULL ws_bytes, short or NULL workspace, NULL row_ptr / col_idx, L == 0 a no-op,
    # at most 2^24 - 1 block rows
    with pytest.raises(sd.SdattnError, match="UNSUPPORTED"):
        sd.sdattn_block_split_workspace(p, 96, 128)
    assert lib.sdattn_block_split_workspace(ctypes.byref(p), 64, 64, None) == 1
    wsb = sd.sdattn_block_split_workspace(p, 64, 64)
    rows = 28 * 256
    assert wsb >= (3 * rows + 2 * 1024 + 2) * 4 + 2 * 1024 * 64 * 129 * 4
    assert sd.sdattn_block_split_workspace(p, 128, 64) >= 2 * 512 * 128 * 129 * 4
    assert lib.sdattn_block_split_plan(ctypes.byref(p), 64, 64, None, BAD, wsb, None) == 1
    assert lib.sdattn_block_split_plan(ctypes.byref(p), 64, 64, BAD, BAD, wsb - 4, None) == 5
    assert lib.sdattn_block_split_plan(ctypes.byref(p), 64, 64, BAD, None, wsb, None) == 5
    assert lib.sdattn_block_split_plan(ctypes.byref(p), 64, 96, BAD, BAD, wsb, None) == 8
    assert lib.sdattn_forward_block_sparse_split(ctypes.byref(p), BAD, BAD, BAD, 64, 64, BAD, None, BAD, wsb, BAD,
                                                 None, None) == 1
    assert lib.sdattn_forward_block_sparse_split(ctypes.byref(p), BAD, BAD, BAD, 64, 64, BAD, BAD, BAD, wsb - 4, BAD,
                                                 None, None) == 5
    assert lib.sdattn_forward_block_sparse_split(ctypes.byref(p), BAD, BAD, BAD, 64, 64, BAD, BAD, BAD, wsb, None,
                                                 None, None) == 1
    assert lib.sdattn_forward_block_sparse_split(ctypes.byref(p), BAD, BAD, BAD, 128, 96, BAD, BAD, BAD, wsb, BAD,
                                                 None, None) == 8
    assert sd.sdattn_block_split_workspace(p0, 64, 64) == 0
    assert lib.sdattn_block_split_plan(ctypes.byref(p0), 64, 64, None, None, 0, None) == 0
    assert lib.sdattn_forward_block_sparse_split(ctypes.byref(p0), None, None, None, 64, 64, None, None, None, 0,
                                                 None, None, None) == 0
    big = sd.problem(8, 64, 64, 1 << 21, 128, "bf16")
    with pytest.raises(sd.SdattnError, match="SHAPE"):
        sd.sdattn_block_split_workspace(big, 64, 64)
    assert lib.sdattn_forward_column_sparse(ctypes.byref(p), BAD, BAD, BAD, BAD, 0, BAD, None, None) == 4
    assert lib.sdattn_forward_column_sparse(ctypes.byref(p), BAD, BAD, BAD, BAD, 16385, BAD, None, None) == 4
    assert lib.sdattn_forward_column_sparse(ctypes.byref(p), BAD, BAD, BAD, None, 492, BAD, None, None) == 1
    ws = sd.sdattn_select_columns_workspace(p, 492)
    assert ws >= 28 * 16384 * 8 + 4 * 16384 * 8
    assert lib.sdattn_select_columns(ctypes.byref(p), BAD, BAD, None, 492, BAD, None, BAD, ws, None) == 1
    assert lib.sdattn_select_columns(ctypes.byref(p), BAD, BAD, BAD, 492, BAD, None, BAD, ws - 8, None) == 5
    with pytest.raises(sd.SdattnError, match="BUDGET"):
        sd.sdattn_select_columns_workspace(p, 0)


def test_exact_selection_validation():
    lib = sd.lib()
    p = sd.problem(1, 4, 4, 4096, 128, "bf16")
    b = sd.topk_budget(0.1)
    ws, nnz = sd.sdattn_select_blocks_exact_workspace(p, 128, 128, b)
    ws_pooled, nnz_pooled = sd.sdattn_select_blocks_workspace(p, 128, 128, b)
    assert nnz == nnz_pooled == 4 * 32 * 4 and ws >= ws_pooled + 4 * 32 * 32 * 4
    sel = lib.sdattn_select_blocks_exact
    assert sel(ctypes.byref(p), BAD, BAD, None, 128, 128, ctypes.byref(b), BAD, BAD, nnz, None, BAD, ws, None) == 1
    assert sel(ctypes.byref(p), BAD, BAD, BAD, 128, 128, ctypes.byref(b), BAD, BAD, nnz - 1, None, BAD, ws, None) == 6
    assert sel(ctypes.byref(p), BAD, BAD, BAD, 128, 128, ctypes.byref(b), BAD, BAD, nnz, None, BAD, ws - 4, None) == 5
    assert sel(ctypes.byref(p), BAD, BAD, BAD, 96, 128, ctypes.byref(b), BAD, BAD, nnz, None, BAD, ws, None) == 8
    with pytest.raises(sd.SdattnError, match="BUDGET"):
        sd.sdattn_select_blocks_exact_workspace(p, 128, 128, sd.topk_budget(0.0))


def test_exact_selection_of_an_empty_sequence_is_a_no_op():
    lib = sd.lib()
    p = sd.problem(1, 4, 4, 0, 128, "bf16")
    b = sd.topk_budget(0.1)
    ws, nnz = sd.sdattn_select_blocks_exact_workspace(p, 128, 128, b)
    assert ws == 0 and nnz == 0
    # nothing is enqueued for L = 0, so NULL buffers are accepted
    assert lib.sdattn_select_blocks_exact(ctypes.byref(p), None, None, None, 128, 128, ctypes.byref(b), None, None,
                                          0, None, None, 0, None) == 0


def test_mask_overlap_validation():
    lib = sd.lib()
    assert lib.sdattn_mask_overlap(-1, BAD, BAD, BAD, BAD, BAD, None) == 2
    assert lib.sdattn_mask_overlap(4, BAD, BAD, BAD, BAD, None, None) == 1
    assert lib.sdattn_mask_overlap(4, BAD, None, BAD, BAD, BAD, None) == 1
    assert lib.sdattn_mask_overlap(4, BAD, BAD, None, BAD, BAD, None) == 1
    assert "non-NULL" in sd.sdattn_last_error()


def test_schedule_descriptor_validation():
    p = sd.problem(1, 4, 4, 512, 64, "f32")
    bad = [
        sd.schedule_desc(10, 2, 5),                                 # select after the warm-up ends
        sd.schedule_desc(0, 0, 0),                                  # no steps
        sd.schedule_desc(10, 1, 0, sel=sd.SDATTN_SEL_COLUMNS, column_keep_frac=0.1),  # columns need refresh_dense
        sd.schedule_desc(10, 0, 0, refresh_dense=True, sel=sd.SDATTN_SEL_COLUMNS, column_keep_frac=0.1),
        sd.schedule_desc(10, 1, 0, block_q=32, block_k=64, budget=sd.topk_budget(0.25)),
    ]
    for d in bad:
        with pytest.raises(sd.SdattnError):
            sd.sdattn_schedule_create(p, d)


def test_header_and_library_from_plain_c(tmp_path):
    """The public header compiles as C99 and as C++17 with warnings as errors,
    and a C program linked against the library gets the same host-side
    answers as the binding."""
    inc = os.path.join(ROOT, "include")
    src = os.path.join(ROOT, "tests", "host", "abi_c_client.c")
    libdir = os.path.dirname(sd.LIB_PATH)
    exe = str(tmp_path / "abi_c_client")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", inc, src, "-o", exe, "-L", libdir,
                    "-lsdattn", f"-Wl,-rpath,{libdir}"], check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert f"C client OK (ABI {sd.SDATTN_ABI_VERSION})" in r.stdout
    cpp = tmp_path / "hdr.cpp"
    cpp.write_text('#include "sdattn.h"\nint main() { return sdattn_abi_version() == SDATTN_ABI_VERSION ? 0 : 1; }\n')
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-I", inc, str(cpp)],
                   check=True, capture_output=True, text=True)


def test_losa_validation():
    """The block-wise (LoSA-style) entry points reject bad problems and
    missing pointers on the host, and size their workspace."""
    lib = sd.lib()
    ws, cap = ctypes.c_size_t(0), ctypes.c_int32(0)
    good = sd.losa_problem(1, 32, 8, 32768, 32, 128, 16, 8, 8)
    assert lib.sdattn_losa_workspace(ctypes.byref(good), ctypes.byref(ws), ctypes.byref(cap)) == 0
    assert cap.value == min(2048, 4 * 8 * 8) and ws.value > 0
    assert lib.sdattn_losa_workspace(None, ctypes.byref(ws), ctypes.byref(cap)) == 1
    assert lib.sdattn_losa_workspace(ctypes.byref(good), None, ctypes.byref(cap)) == 1
    cases = [
        (sd.losa_problem(1, 32, 5, 32768, 32, 128, 16, 8, 8), 2),      # Hq % Hkv
        (sd.losa_problem(0, 32, 8, 32768, 32, 128, 16, 8, 8), 2),      # batch
        (sd.losa_problem(1, 32, 8, 32768, 65, 128, 16, 8, 8), 2),      # block_len > 64
        (sd.losa_problem(1, 32, 8, 32760, 32, 128, 16, 8, 8), 2),      # page does not divide prefix_len
        (sd.losa_problem(1, 32, 8, 131072, 32, 128, 16, 8, 8), 2),     # more than 4096 pages
        (sd.losa_problem(1, 32, 8, 32768, 32, 96, 16, 8, 8), 8),       # head_dim
        (sd.losa_problem(1, 32, 8, 32768, 32, 128, 16, 8, 8, "f32"), 8),
        (sd.losa_problem(1, 32, 8, 32768, 32, 128, 16, 8, 8, 7), 3),   # dtype
        (sd.losa_problem(1, 32, 8, 32768, 32, 128, 16, 0, 8), 4),      # n_active
        (sd.losa_problem(1, 32, 8, 32768, 32, 128, 16, 33, 8), 4),
        (sd.losa_problem(1, 32, 8, 32768, 32, 128, 16, 8, 0), 4),      # pages_per_query
        (sd.losa_problem(1, 32, 8, 32768, 32, 128, 16, 8, 2049), 4),
        (sd.losa_problem(1, 32, 8, 32768, 32, 128, 16, 8, 8, "bf16", float("inf")), 2),
        # 2^24 (batch, query head, Active token) rows: below the old 2^31 bound, but the top-k
        # launch would need 2^32 work-items
        (sd.losa_problem(2048, 256, 8, 4096, 64, 64, 16, 32, 8), 2),
    ]
    for p, code in cases:
        assert lib.sdattn_losa_workspace(ctypes.byref(p), ctypes.byref(ws), ctypes.byref(cap)) == code, \
            sd.sdattn_last_error()
        assert lib.sdattn_losa_pool_pages(ctypes.byref(p), BAD, BAD, None) == code
    # missing pointers and a short workspace fail before any launch
    assert lib.sdattn_losa_pool_pages(ctypes.byref(good), None, BAD, None) == 1
    assert lib.sdattn_losa_dense(ctypes.byref(good), BAD, BAD, BAD, BAD, BAD, BAD, None, BAD, 1 << 40, None) == 1
    assert lib.sdattn_losa_dense(ctypes.byref(good), BAD, BAD, BAD, BAD, BAD, BAD, BAD, BAD, 16, None) == 5
    step = [BAD] * 12
    assert lib.sdattn_losa_step(ctypes.byref(good), *step, None, None, BAD, ctypes.c_size_t(16), None) == 5
    step_missing = list(step)
    step_missing[10] = None  # union_pages
    assert lib.sdattn_losa_step(ctypes.byref(good), *step_missing, None, None, BAD, ctypes.c_size_t(1 << 40),
                                None) == 1
    assert "union_pages" in sd.sdattn_last_error()
    # one row fewer than 2^24 at the same shape passes the launch bounds
    near = sd.losa_problem(2047, 256, 8, 4096, 64, 64, 16, 32, 8)
    assert lib.sdattn_losa_workspace(ctypes.byref(near), ctypes.byref(ws), ctypes.byref(cap)) == 0, \
        sd.sdattn_last_error()
