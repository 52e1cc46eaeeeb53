"""fp64 pattern selection — test infrastructure only (see package header).

Block patterns (SparseD abstract: head-specific patterns computed once;
Step-dLLM abstract: block-sparse mask, uniform or head-adaptive budget):

  1. mean-pool each block of bq query tokens and bk key tokens:
        Qp[h, I] = mean_{i in I} q_i,   Kp[g, J] = mean_{j in J} k_j
     (a last, partial block is the mean of the tokens it has);
  2. pooled scores P[h, I, J] = scale * <Qp[h, I], Kp[g(h), J]>;
  3. pooled mass A[h, I, :] = softmax over J of P[h, I, :];
  4. per row (h, I), order the key blocks by (A descending, J ascending) and
       * top-k: keep the first k = max(1, ceil(rho * nKB)) blocks, or
       * mass with a global cap: keep the shortest prefix whose cumulative
         mass reaches tau*, where tau* is the largest threshold not above the
         mass target for which the mean kept fraction over all rows stays
         within the cap (the head-adaptive global budget: heads whose mass is
         concentrated need fewer blocks to reach the same threshold);
     and list the kept blocks of each row in ascending J (CSR).

Column patterns (PulseCol abstract: column-sparse structure identified from
column-summed attention at an early step):

  C[g, j] = sum over query heads h of group g and all query rows i of the full
            attention probability exp(s_ij - lse_i);
  keep the top kcol = max(1, ceil(rho * L)) columns by (C desc, j asc),
  listed in ascending j.

Ties are broken toward the lower index everywhere.
"""

from fractions import Fraction

import numpy as np

from .attention import as_f64, default_scale, head_group


def count_from_fraction(frac, n: int) -> int:
    """max(1, ceil(frac * n)) clamped to n, with frac read as the decimal it
    was written as (so 0.1 * 10 is exactly 1)."""
    k = Fraction(str(frac)) * n
    k = -((-k.numerator) // k.denominator)  # ceil
    return int(min(n, max(1, k)))


def pool_blocks(x, block: int) -> np.ndarray:
    """Mean of each block of `block` consecutive tokens: [B, H, L, d] -> [B, H, nb, d]."""
    x = as_f64(x)
    B, H, L, d = x.shape
    nb = -(-L // block)
    out = np.zeros((B, H, nb, d))
    for I in range(nb):
        seg = x[:, :, I * block:min(L, (I + 1) * block)]
        out[:, :, I] = seg.sum(axis=2) / seg.shape[2]
    return out


def pooled_scores(q, k, block_q: int, block_k: int, scale=None) -> np.ndarray:
    """P[b, h, I, J] = scale * <Qp[b, h, I], Kp[b, g(h), J]>."""
    qp = pool_blocks(q, block_q)
    kp = pool_blocks(k, block_k)
    B, Hq, nqb, d = qp.shape
    grp = head_group(Hq, kp.shape[1])
    scale = default_scale(d) if scale is None else scale
    return scale * np.einsum("bhid,bhjd->bhij", qp, kp[:, grp])


def pooled_mass(q, k, block_q: int, block_k: int, scale=None) -> np.ndarray:
    """A = softmax over J of the pooled scores: [B, Hq, nQB, nKB]."""
    p = pooled_scores(q, k, block_q, block_k, scale)
    e = np.exp(p - p.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def rank_order(a: np.ndarray) -> np.ndarray:
    """Indices of a 1-D array ordered by (value descending, index ascending)."""
    a = np.asarray(a, dtype=np.float64)
    return np.lexsort((np.arange(len(a)), -a))


def _to_csr(kept_rows):
    counts = np.array([len(r) for r in kept_rows], dtype=np.int64)
    row_ptr = np.zeros(len(kept_rows) + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    col_idx = (np.concatenate([np.sort(r) for r in kept_rows]) if len(kept_rows)
               else np.zeros(0, dtype=np.int64))
    return row_ptr.astype(np.int32), col_idx.astype(np.int32)


def select_topk(A: np.ndarray, keep_frac: float):
    """Top-k block selection per row.  A [B, Hq, nQB, nKB] -> (row_ptr, col_idx)."""
    n = A.shape[-1]
    rows = A.reshape(-1, n)
    k = count_from_fraction(keep_frac, n)
    return _to_csr([rank_order(r)[:k] for r in rows])


def mass_prefix_counts(A: np.ndarray, tau: float) -> np.ndarray:
    """Per row, the length of the shortest (A desc, J asc) prefix whose
    cumulative mass is >= tau (all of the row if no prefix reaches it)."""
    n = A.shape[-1]
    rows = A.reshape(-1, n)
    out = np.empty(len(rows), dtype=np.int64)
    for r, a in enumerate(rows):
        c = np.cumsum(a[rank_order(a)])
        hit = np.nonzero(c >= tau)[0]
        out[r] = hit[0] + 1 if len(hit) else n
    return out


def select_mass_cap(A: np.ndarray, mass: float, max_mean_density: float):
    """Mass budget with a global cap on the mean kept fraction.

    tau* = mass if the mean kept fraction at tau = mass is within the cap;
    otherwise the largest candidate threshold (a cumulative-mass value of some
    row, or the mass target itself) not above the mass target whose mean kept
    fraction is within the cap.  Every row keeps its shortest prefix reaching
    tau*, and at least one block.

    Returns (row_ptr, col_idx, tau_star).
    """
    n = A.shape[-1]
    rows = A.reshape(-1, n)
    R = len(rows)
    cap_total = Fraction(str(max_mean_density)) * R * n  # allowed sum of counts

    def fits(tau):
        return Fraction(int(mass_prefix_counts(A, tau).sum())) <= cap_total

    if fits(mass):
        tau_star = float(mass)
    else:
        cums = np.concatenate([np.cumsum(a[rank_order(a)]) for a in rows])
        cand = np.unique(np.concatenate([cums[cums <= mass], [mass]]))
        lo, hi = 0, len(cand) - 1          # D is non-decreasing in tau
        if not fits(cand[0]):
            tau_star = float(cand[0])      # nothing fits: every row keeps one block
        else:
            while lo < hi:                 # largest index whose threshold fits
                mid = (lo + hi + 1) // 2
                if fits(cand[mid]):
                    lo = mid
                else:
                    hi = mid - 1
            tau_star = float(cand[lo])
    counts = np.maximum(1, mass_prefix_counts(A, tau_star))
    kept = [rank_order(a)[:c] for a, c in zip(rows, counts)]
    row_ptr, col_idx = _to_csr(kept)
    return row_ptr, col_idx, tau_star


def column_scores(q, k, lse, scale=None) -> np.ndarray:
    """C[b, g, j] = sum_{h in group g} sum_i exp(scale <q_i, k_j> - lse_i),
    with lse the log-sum-exp of the full attention rows.  [B, Hkv, L]."""
    q, k = as_f64(q), as_f64(k)
    lse = np.asarray(lse, dtype=np.float64)
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    grp = head_group(Hq, Hkv)
    scale = default_scale(d) if scale is None else scale
    C = np.zeros((B, Hkv, k.shape[2]))
    for b in range(B):
        for h in range(Hq):
            g = grp[h]
            for c0 in range(0, L, 512):
                s = scale * (q[b, h, c0:c0 + 512] @ k[b, g].T)
                C[b, g] += np.exp(s - lse[b, h, c0:c0 + 512, None]).sum(axis=0)
    return C


def exact_block_mass(q, k, lse, block_q: int, block_k: int, scale=None) -> np.ndarray:
    """Exact attention mass of each block pair: the mean over the queries of
    query block I of the probability they give to the keys of key block J,
    A[b, h, I, J] = (1/|I|) sum_{i in I} sum_{j in J} exp(scale <q_i, k_j> - lse_i),
    with lse the log-sum-exp of the full attention rows.  [B, Hq, nQB, nKB].
    (The other reading of a block's attention mass beside the pooled one:
    SparseD, abstract; Step-dLLM, Abstract.)"""
    q, k = as_f64(q), as_f64(k)
    lse = np.asarray(lse, dtype=np.float64)
    B, Hq, L, d = q.shape
    Lk = k.shape[2]
    grp = head_group(Hq, k.shape[1])
    scale = default_scale(d) if scale is None else scale
    nqb, nkb = -(-L // block_q), -(-Lk // block_k)
    A = np.zeros((B, Hq, nqb, nkb))
    for b in range(B):
        for h in range(Hq):
            for I in range(nqb):
                rows = slice(I * block_q, min(L, (I + 1) * block_q))
                P = np.exp(scale * (q[b, h, rows] @ k[b, grp[h]].T) - lse[b, h, rows, None])
                for J in range(nkb):
                    A[b, h, I, J] = P[:, J * block_k:(J + 1) * block_k].sum() / P.shape[0]
    return A


def select_columns(C: np.ndarray, kcol: int) -> np.ndarray:
    """Top-kcol columns per (b, g) by (C desc, j asc), listed ascending.  [B, Hkv, kcol]."""
    B, Hkv, L = C.shape
    if not 1 <= kcol <= L:
        raise ValueError(f"kcol={kcol} outside [1, {L}]")
    out = np.zeros((B, Hkv, kcol), dtype=np.int32)
    for b in range(B):
        for g in range(Hkv):
            out[b, g] = np.sort(rank_order(C[b, g])[:kcol])
    return out
