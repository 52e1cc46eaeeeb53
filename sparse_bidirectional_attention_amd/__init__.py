"""Python binding of libsdattn.so (sparse bidirectional attention, gfx950).

A thin ctypes layer: every function below has the name of the C entry point
it calls and only marshals arguments (torch tensors become device pointers,
the current torch stream becomes the HIP stream).  All compute runs in the
library's HIP kernels.  Importing works without a GPU; calling a compute
entry point needs the built library and a GPU, and raises if either is
missing.

Layout: q, o [B, Hq, L, d]; k, v [B, Hkv, L, d]; lse [B, Hq, L] float32.
"""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsdattn.so")

# ABI of include/sdattn.h that this binding marshals for (SDATTN_ABI_VERSION)
SDATTN_ABI_VERSION = 6

# ---- enums ------------------------------------------------------------------
SDATTN_OK = 0
STATUS_NAMES = ["SDATTN_OK", "SDATTN_ERR_NULL", "SDATTN_ERR_SHAPE", "SDATTN_ERR_DTYPE", "SDATTN_ERR_BUDGET",
                "SDATTN_ERR_WORKSPACE", "SDATTN_ERR_CAPACITY", "SDATTN_ERR_HIP", "SDATTN_ERR_UNSUPPORTED",
                "SDATTN_ERR_STATE"]
SDATTN_F32, SDATTN_BF16 = 0, 1
SDATTN_BUDGET_TOPK, SDATTN_BUDGET_MASS = 0, 1
SDATTN_SEL_BLOCKS, SDATTN_SEL_COLUMNS, SDATTN_SEL_BLOCKS_EXACT = 0, 1, 2
# bytes of the static scratch behind sdattn_select_blocks_noalloc (SDATTN_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20
SEL_KINDS = {"blocks": SDATTN_SEL_BLOCKS, "columns": SDATTN_SEL_COLUMNS, "blocks_exact": SDATTN_SEL_BLOCKS_EXACT}
ACTIONS = ("DENSE", "DENSE_SELECT", "SELECT_SPARSE", "SPARSE", "PROBE_SPARSE")


class SdattnError(RuntimeError):
    def __init__(self, status, where, detail):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{where}: {name}: {detail}")


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int),
                ("softmax_scale", ctypes.c_float)]


class Budget(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("keep_frac", ctypes.c_double), ("mass", ctypes.c_double),
                ("max_mean_density", ctypes.c_double)]


class ScheduleDesc(ctypes.Structure):
    _fields_ = [("total_steps", ctypes.c_int32), ("dense_steps", ctypes.c_int32), ("select_step", ctypes.c_int32),
                ("refresh_interval", ctypes.c_int32), ("refresh_steps", ctypes.POINTER(ctypes.c_int32)),
                ("n_refresh_steps", ctypes.c_int32), ("refresh_dense", ctypes.c_int32), ("sel", ctypes.c_int),
                ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32), ("budget", Budget),
                ("column_keep_frac", ctypes.c_double), ("probe_interval", ctypes.c_int32),
                ("min_overlap", ctypes.c_double), ("split_rows", ctypes.c_int32)]


class LosaProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("prefix_len", ctypes.c_int32), ("block_len", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int), ("softmax_scale", ctypes.c_float), ("page", ctypes.c_int32),
                ("n_active", ctypes.c_int32), ("pages_per_query", ctypes.c_int32)]


_P = ctypes.c_void_p
_SIGS = {
    "sdattn_abi_version": (ctypes.c_int, []),
    "sdattn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sdattn_last_error": (ctypes.c_char_p, []),
    "sdattn_forward_dense": (ctypes.c_int, [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P]),
    "sdattn_select_blocks_workspace": (ctypes.c_int, [ctypes.POINTER(Problem), ctypes.c_int32, ctypes.c_int32,
                                                      ctypes.POINTER(Budget), ctypes.POINTER(ctypes.c_size_t),
                                                      ctypes.POINTER(ctypes.c_int64)]),
    "sdattn_select_blocks": (ctypes.c_int, [ctypes.POINTER(Problem), _P, _P, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.POINTER(Budget), _P, _P, ctypes.c_int64, _P, _P, ctypes.c_size_t,
                                            _P]),
    "sdattn_select_blocks_noalloc": (ctypes.c_int, [ctypes.POINTER(Problem), _P, _P, ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.POINTER(Budget), _P, _P, ctypes.c_int64, _P, _P]),
    "sdattn_select_blocks_exact_workspace": (ctypes.c_int, [ctypes.POINTER(Problem), ctypes.c_int32, ctypes.c_int32,
                                                            ctypes.POINTER(Budget), ctypes.POINTER(ctypes.c_size_t),
                                                            ctypes.POINTER(ctypes.c_int64)]),
    "sdattn_select_blocks_exact": (ctypes.c_int, [ctypes.POINTER(Problem), _P, _P, _P, ctypes.c_int32, ctypes.c_int32,
                                                  ctypes.POINTER(Budget), _P, _P, ctypes.c_int64, _P, _P,
                                                  ctypes.c_size_t, _P]),
    "sdattn_forward_block_sparse": (ctypes.c_int, [ctypes.POINTER(Problem), _P, _P, _P, ctypes.c_int32,
                                                   ctypes.c_int32, _P, _P, _P, _P, _P]),
    "sdattn_block_plan": (ctypes.c_int, [ctypes.POINTER(Problem), ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "sdattn_forward_block_sparse_planned": (ctypes.c_int, [ctypes.POINTER(Problem), _P, _P, _P, ctypes.c_int32,
                                                           ctypes.c_int32, _P, _P, _P, _P, _P, _P]),
    "sdattn_block_split_workspace": (ctypes.c_int, [ctypes.POINTER(Problem), ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.POINTER(ctypes.c_size_t)]),
    "sdattn_block_split_plan": (ctypes.c_int, [ctypes.POINTER(Problem), ctypes.c_int32, ctypes.c_int32, _P, _P,
                                               ctypes.c_size_t, _P]),
    "sdattn_forward_block_sparse_split": (ctypes.c_int, [ctypes.POINTER(Problem), _P, _P, _P, ctypes.c_int32,
                                                         ctypes.c_int32, _P, _P, _P, ctypes.c_size_t, _P, _P, _P]),
    "sdattn_select_columns_workspace": (ctypes.c_int, [ctypes.POINTER(Problem), ctypes.c_int32,
                                                       ctypes.POINTER(ctypes.c_size_t)]),
    "sdattn_select_columns": (ctypes.c_int, [ctypes.POINTER(Problem), _P, _P, _P, ctypes.c_int32, _P, _P, _P,
                                             ctypes.c_size_t, _P]),
    "sdattn_forward_column_sparse": (ctypes.c_int, [ctypes.POINTER(Problem), _P, _P, _P, _P, ctypes.c_int32, _P,
                                                    _P, _P]),
    "sdattn_gather_columns": (ctypes.c_int, [ctypes.POINTER(Problem), _P, _P, _P, ctypes.c_int32, _P, _P, _P]),
    "sdattn_forward_column_packed": (ctypes.c_int, [ctypes.POINTER(Problem), _P, _P, _P, ctypes.c_int32, _P, _P,
                                                    _P]),
    "sdattn_mask_overlap": (ctypes.c_int, [ctypes.c_int32, _P, _P, _P, _P, _P, _P]),
    "sdattn_schedule_create": (ctypes.c_int, [ctypes.POINTER(Problem), ctypes.POINTER(ScheduleDesc),
                                              ctypes.POINTER(_P)]),
    "sdattn_schedule_action": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.POINTER(ctypes.c_int)]),
    "sdattn_schedule_step": (ctypes.c_int, [_P, ctypes.c_int32, _P, _P, _P, _P, _P, _P]),
    "sdattn_schedule_mask": (ctypes.c_int, [_P, ctypes.POINTER(_P), ctypes.POINTER(_P),
                                            ctypes.POINTER(ctypes.c_int64)]),
    "sdattn_schedule_stats": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)]),
    "sdattn_schedule_probe_stats": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                                   ctypes.POINTER(ctypes.c_double), _P]),
    "sdattn_schedule_destroy": (None, [_P]),
    "sdattn_losa_workspace": (ctypes.c_int, [ctypes.POINTER(LosaProblem), ctypes.POINTER(ctypes.c_size_t),
                                             ctypes.POINTER(ctypes.c_int32)]),
    "sdattn_losa_pool_pages": (ctypes.c_int, [ctypes.POINTER(LosaProblem), _P, _P, _P]),
    "sdattn_losa_dense": (ctypes.c_int, [ctypes.POINTER(LosaProblem), _P, _P, _P, _P, _P, _P, _P, _P,
                                         ctypes.c_size_t, _P]),
    "sdattn_losa_step": (ctypes.c_int, [ctypes.POINTER(LosaProblem), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                        _P, _P, _P, _P, ctypes.c_size_t, _P]),
}

_lib_handle = None


def declare(lib, required=True):
    """Attach argument/return types of the C entry points to a ctypes CDLL
    (with required=False, entry points the library lacks are skipped)."""
    for name, (res, args) in _SIGS.items():
        try:
            f = getattr(lib, name)
        except AttributeError:
            if required:
                raise
            continue
        f.restype = res
        f.argtypes = args
    return lib


def lib():
    """The loaded libsdattn.so; raises if it has not been built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m sparse_bidirectional_attention_amd.build`")
        _lib_handle = declare(ctypes.CDLL(LIB_PATH))
    return _lib_handle


def _check(status, where):
    if status != SDATTN_OK:
        detail = lib().sdattn_last_error().decode(errors="replace")
        raise SdattnError(status, where, detail)


def _ptr(x):
    """Device pointer of a torch tensor (or an int / None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError("tensors passed to the library must be on the GPU")
    if not x.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def problem(batch, q_heads, kv_heads, seq_len, head_dim, dtype, softmax_scale=0.0) -> Problem:
    """Problem descriptor; dtype is SDATTN_F32/SDATTN_BF16 or "f32"/"bf16" or a torch dtype."""
    if not isinstance(dtype, int):
        s = str(dtype)
        dtype = SDATTN_BF16 if "bf16" in s or "bfloat16" in s else SDATTN_F32
    return Problem(batch, q_heads, kv_heads, seq_len, head_dim, dtype, softmax_scale)


def problem_of(q, k, softmax_scale=0.0) -> Problem:
    B, Hq, L, d = q.shape
    return problem(B, Hq, k.shape[1], L, d, q.dtype, softmax_scale)


def topk_budget(keep_frac) -> Budget:
    return Budget(SDATTN_BUDGET_TOPK, keep_frac, 0.0, 1.0)


def mass_budget(mass, max_mean_density=1.0) -> Budget:
    return Budget(SDATTN_BUDGET_MASS, 0.0, mass, max_mean_density)


# ---- entry points ---------------------------------------------------------------

def sdattn_abi_version():
    return lib().sdattn_abi_version()


def sdattn_status_string(status):
    return lib().sdattn_status_string(status).decode()


def sdattn_last_error():
    return lib().sdattn_last_error().decode(errors="replace")


def sdattn_forward_dense(p, q, k, v, o, lse=None, stream=None):
    _check(lib().sdattn_forward_dense(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                      _stream(stream)), "sdattn_forward_dense")


def sdattn_select_blocks_workspace(p, block_q, block_k, budget):
    ws = ctypes.c_size_t(0)
    nnz = ctypes.c_int64(0)
    _check(lib().sdattn_select_blocks_workspace(ctypes.byref(p), block_q, block_k, ctypes.byref(budget),
                                                ctypes.byref(ws), ctypes.byref(nnz)),
           "sdattn_select_blocks_workspace")
    return ws.value, nnz.value


def sdattn_select_blocks(p, q, k, block_q, block_k, budget, row_ptr, col_idx, col_capacity=None,
                         block_mass=None, ws=None, ws_bytes=None, stream=None):
    if col_capacity is None:
        col_capacity = col_idx.numel()
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sdattn_select_blocks(ctypes.byref(p), _ptr(q), _ptr(k), block_q, block_k, ctypes.byref(budget),
                                      _ptr(row_ptr), _ptr(col_idx), col_capacity, _ptr(block_mass), _ptr(ws),
                                      ws_bytes, _stream(stream)), "sdattn_select_blocks")


def sdattn_select_blocks_noalloc(p, q, k, block_q, block_k, budget, row_ptr, col_idx, col_capacity=None,
                                 block_mass=None, stream=None):
    """sdattn_select_blocks with the library's static scratch as workspace
    (no allocation; NOALLOC_SCRATCH_BYTES at most)."""
    if col_capacity is None:
        col_capacity = col_idx.numel()
    _check(lib().sdattn_select_blocks_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), block_q, block_k,
                                              ctypes.byref(budget), _ptr(row_ptr), _ptr(col_idx), col_capacity,
                                              _ptr(block_mass), _stream(stream)), "sdattn_select_blocks_noalloc")


def sdattn_select_blocks_exact_workspace(p, block_q, block_k, budget):
    ws = ctypes.c_size_t(0)
    nnz = ctypes.c_int64(0)
    _check(lib().sdattn_select_blocks_exact_workspace(ctypes.byref(p), block_q, block_k, ctypes.byref(budget),
                                                      ctypes.byref(ws), ctypes.byref(nnz)),
           "sdattn_select_blocks_exact_workspace")
    return ws.value, nnz.value


def sdattn_select_blocks_exact(p, q, k, lse, block_q, block_k, budget, row_ptr, col_idx, col_capacity=None,
                               block_mass=None, ws=None, ws_bytes=None, stream=None):
    if col_capacity is None:
        col_capacity = col_idx.numel()
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sdattn_select_blocks_exact(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(lse), block_q, block_k,
                                            ctypes.byref(budget), _ptr(row_ptr), _ptr(col_idx), col_capacity,
                                            _ptr(block_mass), _ptr(ws), ws_bytes, _stream(stream)),
           "sdattn_select_blocks_exact")


def sdattn_forward_block_sparse(p, q, k, v, block_q, block_k, row_ptr, col_idx, o, lse=None, stream=None):
    _check(lib().sdattn_forward_block_sparse(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), block_q, block_k,
                                             _ptr(row_ptr), _ptr(col_idx), _ptr(o), _ptr(lse), _stream(stream)),
           "sdattn_forward_block_sparse")


def sdattn_block_plan(p, block_q, block_k, row_ptr, plan, stream=None):
    """plan: int32 device tensor of B*Hq*nQB entries <- the dispatch plan of row_ptr's pattern."""
    _check(lib().sdattn_block_plan(ctypes.byref(p), block_q, block_k, _ptr(row_ptr), _ptr(plan), _stream(stream)),
           "sdattn_block_plan")


def sdattn_forward_block_sparse_planned(p, q, k, v, block_q, block_k, row_ptr, col_idx, plan, o, lse=None,
                                        stream=None):
    _check(lib().sdattn_forward_block_sparse_planned(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), block_q, block_k,
                                                     _ptr(row_ptr), _ptr(col_idx), _ptr(plan), _ptr(o), _ptr(lse),
                                                     _stream(stream)), "sdattn_forward_block_sparse_planned")


def sdattn_block_split_workspace(p, block_q, block_k):
    ws = ctypes.c_size_t(0)
    _check(lib().sdattn_block_split_workspace(ctypes.byref(p), block_q, block_k, ctypes.byref(ws)),
           "sdattn_block_split_workspace")
    return ws.value


def sdattn_block_split_plan(p, block_q, block_k, row_ptr, ws, ws_bytes=None, stream=None):
    """ws: uint8 device tensor of sdattn_block_split_workspace bytes <- the split plan of row_ptr's pattern."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().sdattn_block_split_plan(ctypes.byref(p), block_q, block_k, _ptr(row_ptr), _ptr(ws), ws_bytes,
                                         _stream(stream)), "sdattn_block_split_plan")


def sdattn_forward_block_sparse_split(p, q, k, v, block_q, block_k, row_ptr, col_idx, ws, o, lse=None,
                                      ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    _check(lib().sdattn_forward_block_sparse_split(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), block_q, block_k,
                                                   _ptr(row_ptr), _ptr(col_idx), _ptr(ws), ws_bytes, _ptr(o),
                                                   _ptr(lse), _stream(stream)), "sdattn_forward_block_sparse_split")


def sdattn_select_columns_workspace(p, kcol):
    ws = ctypes.c_size_t(0)
    _check(lib().sdattn_select_columns_workspace(ctypes.byref(p), kcol, ctypes.byref(ws)),
           "sdattn_select_columns_workspace")
    return ws.value


def sdattn_select_columns(p, q, k, lse, kcol, col_idx, col_scores=None, ws=None, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sdattn_select_columns(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(lse), kcol, _ptr(col_idx),
                                       _ptr(col_scores), _ptr(ws), ws_bytes, _stream(stream)),
           "sdattn_select_columns")


def sdattn_forward_column_sparse(p, q, k, v, col_idx, kcol, o, lse=None, stream=None):
    _check(lib().sdattn_forward_column_sparse(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(col_idx), kcol,
                                              _ptr(o), _ptr(lse), _stream(stream)),
           "sdattn_forward_column_sparse")


def sdattn_gather_columns(p, k, v, col_idx, kcol, kc, vc, stream=None):
    _check(lib().sdattn_gather_columns(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(col_idx), kcol, _ptr(kc), _ptr(vc),
                                       _stream(stream)), "sdattn_gather_columns")


def sdattn_forward_column_packed(p, q, kc, vc, kcol, o, lse=None, stream=None):
    _check(lib().sdattn_forward_column_packed(ctypes.byref(p), _ptr(q), _ptr(kc), _ptr(vc), kcol, _ptr(o), _ptr(lse),
                                              _stream(stream)), "sdattn_forward_column_packed")


def sdattn_mask_overlap(rows, row_ptr_a, col_idx_a, row_ptr_b, col_idx_b, counts, stream=None):
    """counts: int64 device tensor of 3 slots <- (|A n B|, |A|, |B|)."""
    _check(lib().sdattn_mask_overlap(rows, _ptr(row_ptr_a), _ptr(col_idx_a), _ptr(row_ptr_b), _ptr(col_idx_b),
                                     _ptr(counts), _stream(stream)), "sdattn_mask_overlap")


def schedule_desc(total_steps, dense_steps, select_step, refresh_interval=0, refresh_steps=(), refresh_dense=False,
                  sel=SDATTN_SEL_BLOCKS, block_q=128, block_k=128, budget=None, column_keep_frac=0.0,
                  probe_interval=0, min_overlap=0.0, split_rows=False):
    arr = (ctypes.c_int32 * max(1, len(refresh_steps)))(*refresh_steps)
    d = ScheduleDesc(total_steps, dense_steps, select_step, refresh_interval,
                     ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)) if refresh_steps else None,
                     len(refresh_steps), int(bool(refresh_dense)), sel, block_q, block_k,
                     budget if budget is not None else topk_budget(1.0), column_keep_frac, probe_interval,
                     min_overlap, int(bool(split_rows)))
    d._keep = arr  # the C side copies the array at create; keep it alive until then
    return d


def sdattn_schedule_create(p, desc):
    h = ctypes.c_void_p(None)
    _check(lib().sdattn_schedule_create(ctypes.byref(p), ctypes.byref(desc), ctypes.byref(h)),
           "sdattn_schedule_create")
    return h


def sdattn_schedule_action(h, step):
    a = ctypes.c_int(0)
    _check(lib().sdattn_schedule_action(h, step, ctypes.byref(a)), "sdattn_schedule_action")
    return ACTIONS[a.value]


def sdattn_schedule_step(h, step, q, k, v, o, lse=None, stream=None):
    _check(lib().sdattn_schedule_step(h, step, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _stream(stream)),
           "sdattn_schedule_step")


def sdattn_schedule_mask(h):
    rp, ci, cap = ctypes.c_void_p(None), ctypes.c_void_p(None), ctypes.c_int64(0)
    _check(lib().sdattn_schedule_mask(h, ctypes.byref(rp), ctypes.byref(ci), ctypes.byref(cap)),
           "sdattn_schedule_mask")
    return rp.value, ci.value, cap.value


def sdattn_schedule_stats(h):
    counts = (ctypes.c_int64 * 4)()
    last = ctypes.c_int32(0)
    _check(lib().sdattn_schedule_stats(h, counts, ctypes.byref(last)), "sdattn_schedule_stats")
    return {a: counts[i] for i, a in enumerate(ACTIONS[:4])}, last.value


def sdattn_schedule_probe_stats(h, stream=None):
    """(probe steps run, probes adopted, overlap of the last probe); waits for the stream."""
    n, a, j = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_double(0.0)
    _check(lib().sdattn_schedule_probe_stats(h, ctypes.byref(n), ctypes.byref(a), ctypes.byref(j), _stream(stream)),
           "sdattn_schedule_probe_stats")
    return n.value, a.value, j.value


def sdattn_schedule_destroy(h):
    lib().sdattn_schedule_destroy(h)


# ---- block-wise diffusion over a cached prefix (LoSA-style) ----------------

def losa_problem(batch, q_heads, kv_heads, prefix_len, block_len, head_dim, page, n_active, pages_per_query,
                 dtype="bf16", softmax_scale=0.0):
    dt = {"f32": SDATTN_F32, "bf16": SDATTN_BF16}[dtype] if isinstance(dtype, str) else int(dtype)
    return LosaProblem(batch, q_heads, kv_heads, prefix_len, block_len, head_dim, dt, softmax_scale, page, n_active,
                       pages_per_query)


def sdattn_losa_workspace(p):
    """Returns (ws_bytes, max_union_pages)."""
    ws = ctypes.c_size_t(0)
    cap = ctypes.c_int32(0)
    _check(lib().sdattn_losa_workspace(ctypes.byref(p), ctypes.byref(ws), ctypes.byref(cap)), "sdattn_losa_workspace")
    return ws.value, cap.value


def sdattn_losa_pool_pages(p, k_cache, kp, stream=None):
    _check(lib().sdattn_losa_pool_pages(ctypes.byref(p), _ptr(k_cache), _ptr(kp), _stream(stream)),
           "sdattn_losa_pool_pages")


def sdattn_losa_dense(p, q, k_cache, v_cache, k_blk, v_blk, o, lse, ws, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sdattn_losa_dense(ctypes.byref(p), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_blk), _ptr(v_blk),
                                   _ptr(o), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)), "sdattn_losa_dense")


def sdattn_losa_step(p, q, q_prev, k_cache, v_cache, kp, k_blk, v_blk, o, lse, active_idx, union_pages, union_count,
                     ws, locality=None, page_scores=None, stream=None):
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sdattn_losa_step(ctypes.byref(p), _ptr(q), _ptr(q_prev), _ptr(k_cache), _ptr(v_cache), _ptr(kp),
                                  _ptr(k_blk), _ptr(v_blk), _ptr(o), _ptr(lse), _ptr(active_idx), _ptr(union_pages),
                                  _ptr(union_count), _ptr(locality), _ptr(page_scores), _ptr(ws), ws_bytes,
                                  _stream(stream)), "sdattn_losa_step")
