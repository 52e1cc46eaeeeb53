"""fp64 LoSA-style partial attention for block-wise diffusion — test infrastructure only.

What is computed (LoSA: Locality Aware Sparse Attention for block-wise
diffusion language models; sections 1 "the problem", 2 "the observation" and
3 "methodology", its core principles and workflow):

A block-wise diffusion LM denoises a block of Bs tokens at a time on top of a
prefix of Lp tokens whose keys and values sit in a cache.  Each query of the
block attends, without a causal mask, to every prefix key and every key of the
block.  On the first iteration of a block that attention is computed densely,
which fills the output cache.  On each later iteration:

  1. locality score of block token i: the mean squared change of its query
     vector since the previous iteration,
         delta_i = mean over (h, c) of (q_t[h, i, c] - q_{t-1}[h, i, c])^2
     (the token's query vector is all query heads side by side);
  2. the n_active tokens with the largest delta_i are Active, the rest Stable
     (ties: lower index first);
  3. a sparse selector runs for the Active tokens only: for query head h and
     Active token i, page P of the prefix (page tokens P*ps .. P*ps+ps-1)
     scores  s[h, i, P] = scale * <q_t[h, i], Kp[g(h), P]>  with Kp the mean
     of the page's cached keys, and the row keeps its top-k pages
     (score descending, page ascending);
  4. the union of the kept pages over the Active tokens and the query heads of
     kv head g is the only part of the prefix loaded for g;
  5. each Active query attends to the prefix tokens of that union (the prefix
     contribution) and to all Bs keys of the block (the suffix contribution),
     and the two are combined by the online-softmax merge; here the oracle
     takes the softmax over both key sets at once, which is what the merge
     must equal;
  6. a Stable token keeps its previous output and log-sum-exp.

Readings where the page is silent (each is listed with the other readings):
  * the locality score averages over all query heads (one Active set per
    token, shared by the heads);
  * Active tokens are a fixed count n_active, not a threshold;
  * the page names QUEST as the selector but does not give it; a mean-pooled
    key per page scored against the single query stands in (the pooling of
    SparseD's selector applied to one query);
  * the union is taken per kv head (the unit of the cache that is loaded),
    and every Active query of the group attends to the whole union.

Shapes: q, q_prev [B, Hq, Bs, d]; k_cache, v_cache [B, Hkv, Lp, d];
k_blk, v_blk [B, Hkv, Bs, d]; o [B, Hq, Bs, d]; lse [B, Hq, Bs].
"""

import numpy as np

from .attention import _attend, as_f64, default_scale, head_group
from .select import pool_blocks, rank_order


def locality_scores(q, q_prev) -> np.ndarray:
    """delta[b, i]: mean over heads and channels of the squared query change."""
    dq = as_f64(q) - as_f64(q_prev)
    B, Hq, Bs, d = dq.shape
    return (dq * dq).transpose(0, 2, 1, 3).reshape(B, Bs, Hq * d).mean(axis=-1)


def select_active(delta, n_active: int) -> np.ndarray:
    """Per batch row, the n_active largest locality scores (ties: lower index
    first), listed ascending.  [B, n_active] int."""
    delta = np.asarray(delta, dtype=np.float64)
    B, Bs = delta.shape
    if not 1 <= n_active <= Bs:
        raise ValueError(f"n_active={n_active} outside [1, {Bs}]")
    return np.stack([np.sort(rank_order(delta[b])[:n_active]) for b in range(B)]).astype(np.int64)


def pool_pages(k_cache, page: int) -> np.ndarray:
    """Kp[b, g, P]: mean of the cached keys of page P.  [B, Hkv, Lp/page, d]."""
    return pool_blocks(k_cache, page)


def page_scores(q, active, kp, scale=None) -> np.ndarray:
    """s[b, h, a, P] = scale * <q[b, h, active[b, a]], Kp[b, g(h), P]>."""
    q, kp = as_f64(q), np.asarray(kp, dtype=np.float64)
    B, Hq, Bs, d = q.shape
    grp = head_group(Hq, kp.shape[1])
    scale = default_scale(d) if scale is None else scale
    n_a = active.shape[1]
    s = np.zeros((B, Hq, n_a, kp.shape[2]))
    for b in range(B):
        for h in range(Hq):
            s[b, h] = scale * (q[b, h, active[b]] @ kp[b, grp[h]].T)
    return s


def select_pages(scores, k: int) -> np.ndarray:
    """Top-k pages of every score row (score descending, page ascending),
    listed ascending.  [B, Hq, n_a, k] int."""
    scores = np.asarray(scores, dtype=np.float64)
    B, Hq, n_a, npg = scores.shape
    if not 1 <= k <= npg:
        raise ValueError(f"pages_per_query={k} outside [1, {npg}]")
    out = np.zeros((B, Hq, n_a, k), dtype=np.int64)
    for b in range(B):
        for h in range(Hq):
            for a in range(n_a):
                out[b, h, a] = np.sort(rank_order(scores[b, h, a])[:k])
    return out


def union_pages(sel, kv_heads: int):
    """Per (b, g): the ascending union of the pages kept by the query heads of
    kv head g over all Active tokens.  Returns a list of lists of int arrays."""
    B, Hq = sel.shape[:2]
    grp = head_group(Hq, kv_heads)
    return [[np.unique(sel[b, grp == g].ravel()) for g in range(kv_heads)] for b in range(B)]


def _concat_keys(k_cache, v_cache, k_blk, v_blk):
    k = np.concatenate([as_f64(k_cache), as_f64(k_blk)], axis=2)
    v = np.concatenate([as_f64(v_cache), as_f64(v_blk)], axis=2)
    return k, v


def block_attention(q, k_cache, v_cache, k_blk, v_blk, allowed_prefix, rows, scale=None):
    """Attention of the query rows `rows[b]` (block token indices) over the
    prefix tokens allowed for their kv head and all keys of the block.

    allowed_prefix: bool [B, Hkv, Lp].  Returns o [B, Hq, len(rows[b]), d],
    lse [B, Hq, len(rows[b])]: the softmax over both key sets at once."""
    q = as_f64(q)
    k, v = _concat_keys(k_cache, v_cache, k_blk, v_blk)
    B, Hq, Bs, d = q.shape
    Hkv, Lp = k_cache.shape[1], k_cache.shape[2]
    grp = head_group(Hq, Hkv)
    scale = default_scale(d) if scale is None else scale
    n = rows.shape[1]
    o = np.zeros((B, Hq, n, v.shape[-1]))
    lse = np.zeros((B, Hq, n))
    for b in range(B):
        for h in range(Hq):
            g = grp[h]
            allowed = np.concatenate([allowed_prefix[b, g], np.ones(Bs, dtype=bool)])
            s = scale * (q[b, h, rows[b]] @ k[b, g].T)
            s = np.where(allowed[None, :], s, -np.inf)
            o[b, h], lse[b, h] = _attend(s, v[b, g])
    return o, lse


def losa_dense(q, k_cache, v_cache, k_blk, v_blk, scale=None):
    """The first iteration of a block: every block query over the whole prefix
    and the whole block.  Returns o [B, Hq, Bs, d], lse [B, Hq, Bs]."""
    B, Hq, Bs, _ = q.shape
    Hkv, Lp = k_cache.shape[1], k_cache.shape[2]
    rows = np.tile(np.arange(Bs), (B, 1))
    return block_attention(q, k_cache, v_cache, k_blk, v_blk, np.ones((B, Hkv, Lp), dtype=bool), rows, scale)


def union_token_mask(unions, Lp: int, page: int) -> np.ndarray:
    """bool [B, Hkv, Lp]: the prefix tokens of each union's pages."""
    B, Hkv = len(unions), len(unions[0])
    m = np.zeros((B, Hkv, Lp), dtype=bool)
    for b in range(B):
        for g in range(Hkv):
            for P in unions[b][g]:
                m[b, g, P * page:(P + 1) * page] = True
    return m


def losa_attention(q, k_cache, v_cache, k_blk, v_blk, active, unions, page, o_prev, lse_prev, scale=None):
    """One later iteration given its Active set and page unions: Active rows
    get the attention over (union tokens of the prefix) + (the block); Stable
    rows keep o_prev / lse_prev.  Returns o, lse (float64)."""
    Lp = k_cache.shape[2]
    o = as_f64(o_prev).copy()
    lse = np.asarray(lse_prev, dtype=np.float64).copy()
    oa, la = block_attention(q, k_cache, v_cache, k_blk, v_blk, union_token_mask(unions, Lp, page), active, scale)
    for b in range(q.shape[0]):
        o[b][:, active[b]] = oa[b]
        lse[b][:, active[b]] = la[b]
    return o, lse


def losa_step(q, q_prev, k_cache, v_cache, k_blk, v_blk, o_prev, lse_prev, page, n_active, pages_per_query,
              scale=None):
    """The whole later iteration from its inputs: locality, Active set, page
    scores, per-row page selection, unions, attention.  Returns a dict."""
    Hkv = k_cache.shape[1]
    delta = locality_scores(q, q_prev)
    active = select_active(delta, n_active)
    kp = pool_pages(k_cache, page)
    s = page_scores(q, active, kp, scale)
    sel = select_pages(s, pages_per_query)
    unions = union_pages(sel, Hkv)
    o, lse = losa_attention(q, k_cache, v_cache, k_blk, v_blk, active, unions, page, o_prev, lse_prev, scale)
    return {"delta": delta, "active": active, "kp": kp, "scores": s, "sel": sel, "unions": unions,
            "o": o, "lse": lse}
