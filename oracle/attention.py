"""fp64 masked softmax attention — test infrastructure only (see package header).

What is computed (SparseD abstract; Step-dLLM abstract; PulseCol abstract):
bidirectional (non-causal) softmax attention of every query over an allowed
set of keys.  Dense attention allows every key; block-sparse attention allows
the key tokens of the kept key blocks of the query's block; column-sparse
attention allows a fixed list of key tokens shared by the query heads of one
key/value head.  Per query row i of head h with allowed set M_i:

    s_ij   = scale * <q_i, k_j>          (k, v from kv head g(h))
    m_i    = max_{j in M_i} s_ij
    l_i    = sum_{j in M_i} exp(s_ij - m_i)
    o_i    = sum_{j in M_i} exp(s_ij - m_i) v_j / l_i
    lse_i  = m_i + ln l_i                (natural log)

An empty allowed set gives o_i = 0 and lse_i = -inf.

Readings where the pages are silent: scale = 1/sqrt(d); query head h reads
kv head floor(h / (Hq/Hkv)) (consecutive groups).
"""

import numpy as np


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns (uint16)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_f64(x) -> np.ndarray:
    """Inputs as float64: uint16 arrays are bf16 bit patterns, others are cast."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return decode_bf16(x)
    return x.astype(np.float64)


def default_scale(d: int) -> float:
    return 1.0 / np.sqrt(d)


def head_group(hq: int, hkv: int) -> np.ndarray:
    """kv head read by each query head: consecutive groups of Hq/Hkv heads."""
    if hkv <= 0 or hq % hkv:
        raise ValueError(f"q_heads={hq} must be a positive multiple of kv_heads={hkv}")
    return np.arange(hq) // (hq // hkv)


def _attend(s: np.ndarray, v: np.ndarray):
    """Softmax over the last axis of scores s (masked entries are -inf), times v.

    s: [n, m] float64, v: [m, d].  Returns o [n, d], lse [n].
    """
    m = s.max(axis=-1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.exp(s - m_safe[:, None])
    l = p.sum(axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        o = np.where(empty[:, None], 0.0, (p @ v) / l[:, None])
        lse = np.where(empty, -np.inf, m_safe + np.log(l))
    return o, lse


def dense_attention(q, k, v, scale=None, rows=None):
    """Full bidirectional attention.

    q [B, Hq, L, d], k/v [B, Hkv, L, d].  `rows` optionally restricts the query
    positions (same for every head).  Returns o [B, Hq, n, d], lse [B, Hq, n].
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    B, Hq, L, d = q.shape
    grp = head_group(Hq, k.shape[1])
    scale = default_scale(d) if scale is None else scale
    rows = np.arange(L) if rows is None else np.asarray(rows)
    o = np.zeros((B, Hq, len(rows), v.shape[-1]))
    lse = np.zeros((B, Hq, len(rows)))
    for b in range(B):
        for h in range(Hq):
            g = grp[h]
            for c0 in range(0, len(rows), 256):
                r = rows[c0:c0 + 256]
                s = scale * (q[b, h, r] @ k[b, g].T)
                o[b, h, c0:c0 + 256], lse[b, h, c0:c0 + 256] = _attend(s, v[b, g])
    return o, lse


def masked_attention(q, k, v, allowed, scale=None):
    """Attention with a token mask, written as the definition: disallowed
    scores are set to -inf before the softmax.

    allowed: bool [B, Hq, L, L] (query i may attend key j).
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    B, Hq, L, d = q.shape
    grp = head_group(Hq, k.shape[1])
    scale = default_scale(d) if scale is None else scale
    o = np.zeros((B, Hq, L, v.shape[-1]))
    lse = np.zeros((B, Hq, L))
    for b in range(B):
        for h in range(Hq):
            g = grp[h]
            s = scale * (q[b, h] @ k[b, g].T)
            s = np.where(allowed[b, h], s, -np.inf)
            o[b, h], lse[b, h] = _attend(s, v[b, g])
    return o, lse


def block_token_mask(row_ptr, col_idx, B, Hq, L, block_q, block_k):
    """Token mask of a CSR block list: row r = (b*Hq + h)*nQB + I lists the
    kept key blocks J of query block I; every query of block I may attend
    every key token of those blocks."""
    nqb = -(-L // block_q)
    allowed = np.zeros((B, Hq, L, L), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            for I in range(nqb):
                r = (b * Hq + h) * nqb + I
                for J in col_idx[row_ptr[r]:row_ptr[r + 1]]:
                    allowed[b, h, I * block_q:(I + 1) * block_q, J * block_k:(J + 1) * block_k] = True
    return allowed


def column_token_mask(col_idx, Hq, L):
    """Token mask of per-kv-head key columns: every query of every query head
    in group g may attend exactly the keys col_idx[b, g, :]."""
    B, Hkv, _ = col_idx.shape
    grp = head_group(Hq, Hkv)
    allowed = np.zeros((B, Hq, L, L), dtype=bool)
    for b in range(B):
        for h in range(Hq):
            allowed[b, h, :, col_idx[b, grp[h]]] = True
    return allowed


def block_sparse_attention(q, k, v, row_ptr, col_idx, block_q, block_k, scale=None, qblocks=None):
    """Block-sparse attention in gather form: each query block attends only
    the key tokens of its kept key blocks.

    row_ptr [B*Hq*nQB + 1], col_idx [nnz] (CSR over rows (b, h, I)).
    `qblocks` optionally restricts the query blocks (same for every head).
    Returns o [B, Hq, n_tokens, d], lse [B, Hq, n_tokens] over the selected
    query blocks' tokens, in block order.
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    B, Hq, L, d = q.shape
    grp = head_group(Hq, k.shape[1])
    scale = default_scale(d) if scale is None else scale
    nqb = -(-L // block_q)
    qblocks = np.arange(nqb) if qblocks is None else np.asarray(qblocks)
    toks = np.concatenate([np.arange(I * block_q, min(L, (I + 1) * block_q)) for I in qblocks])
    o = np.zeros((B, Hq, len(toks), v.shape[-1]))
    lse = np.zeros((B, Hq, len(toks)))
    for b in range(B):
        for h in range(Hq):
            g = grp[h]
            pos = 0
            for I in qblocks:
                r = (b * Hq + h) * nqb + I
                qi = np.arange(I * block_q, min(L, (I + 1) * block_q))
                kept = col_idx[row_ptr[r]:row_ptr[r + 1]]
                kj = (np.concatenate([np.arange(J * block_k, min(L, (J + 1) * block_k)) for J in kept])
                      if len(kept) else np.zeros(0, dtype=np.int64))
                s = scale * (q[b, h, qi] @ k[b, g, kj].T) if len(kj) else np.full((len(qi), 0), -np.inf)
                if len(kj):
                    o[b, h, pos:pos + len(qi)], lse[b, h, pos:pos + len(qi)] = _attend(s, v[b, g, kj])
                else:
                    o[b, h, pos:pos + len(qi)], lse[b, h, pos:pos + len(qi)] = 0.0, -np.inf
                pos += len(qi)
    return o, lse


def column_sparse_attention(q, k, v, col_idx, scale=None, rows=None):
    """Column-sparse attention in gather form: every query of every query head
    of group g attends only the key tokens col_idx[b, g, :] (PulseCol
    abstract: column-level sparsity shared across queries).

    col_idx [B, Hkv, kcol].  `rows` optionally restricts the query positions.
    """
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    B, Hq, L, d = q.shape
    grp = head_group(Hq, k.shape[1])
    scale = default_scale(d) if scale is None else scale
    rows = np.arange(L) if rows is None else np.asarray(rows)
    o = np.zeros((B, Hq, len(rows), v.shape[-1]))
    lse = np.zeros((B, Hq, len(rows)))
    for b in range(B):
        for h in range(Hq):
            g = grp[h]
            cols = np.asarray(col_idx[b, g])
            if len(cols) == 0:
                lse[b, h] = -np.inf
                continue
            s = scale * (q[b, h, rows] @ k[b, g, cols].T)
            o[b, h], lse[b, h] = _attend(s, v[b, g, cols])
    return o, lse
