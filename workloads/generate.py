"""Seeded synthetic Q/K/V with planted, head-varying structure.

The pages measure on activations of real diffusion LMs, which are not
available.  These tensors stand in for them: N(0, 1) entries at the model
shapes, plus planted structure that mimics what the pages observe (patterns
differ across heads and stay similar across steps; heads concentrate their
attention to different extents; SparseD and Step-dLLM abstracts).

Recipe (all draws from numpy PCG64 seeded by SeedSequence):
  * base tensors  : SeedSequence([wid, 0, tensor]) standard normal, fp32.
  * head types    : round-robin by h mod 4 -> sink, local, stripes, none.
      sink    : K of tokens 0..63 += 3u and every Q of the head += 3u.
      local   : unit e_b per 64-token unit; q_i += 3 e_{i//64};
                k_j += 3 normalize(sum_{|c - j//64| <= 2} e_c)  (a +-128 band).
      stripes : K of 4 random 64-token units += 3u and every Q += 3u.
  * extra pairs   : a fraction of (I, J) block pairs per head gets its own unit
                    w; q in block I += 2w, k in block J += 2w.
  * columns       : per kv head g, n random single tokens get K += 3u_g and
                    every Q of the group's query heads += 3u_g.
  * steps         : "fresh_qv": Q_t = Q_0 + s N_t, V_t = V_0 + s N_t, K fixed.
                    "walk": Q_t = Q_0 + s W_t, K_t likewise (independent
                    walks), V fixed, where W is a Gaussian random walk:
                    W_0 = 0 and the increments W_t - W_{t-1} are independent
                    N(0, 1) per element.  W is built by the dyadic (Levy)
                    Brownian-bridge construction on [0, T2], T2 the smallest
                    power of two >= the step count: W_T2 = sqrt(T2) Z_root,
                    and the midpoint c of a dyadic interval [a, b] takes
                    W_c = (W_a + W_b) / 2 + sqrt((b - a) / 4) Z_(a, b).  So
                    any step is a fixed combination of at most log2(T2) + 1
                    seeded standard-normal tensors, computable without
                    replaying the earlier steps, and consecutive steps differ
                    by s N(0, 1) per element.  Each node tensor is drawn in
                    chunks of 2^22 elements, chunk c of node (a, b) of tensor
                    n from SeedSequence([wid, 1000 + n, a, b, c]) (the root
                    is node (T2, T2)).
  * bf16          : the fp32 step tensor rounded to nearest-even.
  * block-wise (LoSA workloads): prefix K/V caches N(0, 1) and a block's Q/K/V
    N(0, 1) from SeedSequence([wid, 0, tensor]); kv head types by g mod 4:
      sink    : K of prefix tokens 0..63 += 3u, the group's block Q += 3u;
      recent  : K of the last 256 prefix tokens += 3u, the group's block Q += 3u;
      stripes : K of 4 random 64-token prefix units += 3u, block Q += 3u;
    and per kv head, each block token i gets its own unit w_i: its group's
    queries += 2 w_i and the keys of pages_per_token random prefix pages
    += 2 w_i, so Active tokens select different pages.  Iteration t >= 1 adds
    sigma_move N to q, k, v of n_moving random block tokens and sigma_still N
    to the others (SeedSequence([wid, 1 + t, 10 + tensor])), accumulated from
    iteration 0.

Tensors are returned as numpy arrays of shape [B, H, L, d]: float32 for the
fp32 workloads, uint16 bf16 bit patterns for the bf16 workloads.
"""

import numpy as np

from .configs import LosaWorkload, Workload

_T_Q, _T_K, _T_V = 0, 1, 2
UNIT = 64  # token unit of the planted sink/local/stripe patterns


def _rng(*key):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def _unit(rng, d):
    x = rng.standard_normal(d)
    return (x / np.linalg.norm(x)).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _plant_mix(w: Workload, q, k):
    """Round-robin head types sink / local / stripes / none (in place, fp32).

    The type is chosen per kv head; the key planting goes to that kv head and the query
    planting to every query head of its group (one head per group without GQA)."""
    B, Hq, L, d = q.shape
    H = k.shape[1]
    G = Hq // H
    n_units = -(-L // UNIT)
    for h in range(H):
        kind = h % 4
        r = _rng(w.wid, 100, h)
        qs = slice(h * G, (h + 1) * G)
        if kind == 0:  # sink
            u = _unit(r, d)
            k[:, h, :min(UNIT, L)] += 3.0 * u
            q[:, qs] += 3.0 * u
        elif kind == 1:  # local band of +-2 units
            e = np.stack([_unit(r, d) for _ in range(n_units)])
            band = np.zeros_like(e)
            for c in range(n_units):
                lo, hi = max(0, c - 2), min(n_units, c + 3)
                s = e[lo:hi].sum(axis=0)
                band[c] = s / np.linalg.norm(s)
            tok_unit = np.arange(L) // UNIT
            q[:, qs] += 3.0 * e[tok_unit]
            k[:, h] += 3.0 * band[tok_unit]
        elif kind == 2:  # vertical stripes: 4 random 64-token units
            u = _unit(r, d)
            units = r.choice(n_units, size=min(4, n_units), replace=False)
            for c in units:
                k[:, h, c * UNIT:min(L, (c + 1) * UNIT)] += 3.0 * u
            q[:, qs] += 3.0 * u


def _plant_pairs(w: Workload, q, k):
    """Extra alignment on a random fraction of (I, J) block pairs per kv head (its query
    group shares the pairs)."""
    B, Hq, L, d = q.shape
    H = k.shape[1]
    G = Hq // H
    nb = -(-L // w.block)
    n_pairs = int(round(w.extra_pair_frac * nb * nb))
    if n_pairs == 0:
        return
    for h in range(H):
        r = _rng(w.wid, 200, h)
        flat = r.choice(nb * nb, size=n_pairs, replace=False)
        wv = r.standard_normal((n_pairs, d))
        wv = (wv / np.linalg.norm(wv, axis=1, keepdims=True)).astype(np.float32)
        qadd = np.zeros((nb, d), np.float32)
        kadd = np.zeros((nb, d), np.float32)
        np.add.at(qadd, flat // nb, 2.0 * wv)
        np.add.at(kadd, flat % nb, 2.0 * wv)
        tok_blk = np.arange(L) // w.block
        q[:, h * G:(h + 1) * G] += qadd[tok_blk][None, None]
        k[:, h] += kadd[tok_blk]


def _plant_columns(w: Workload, q, k):
    """Per kv head, single-token key columns aligned with the group's queries."""
    B, Hq, L, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    for g in range(Hkv):
        r = _rng(w.wid, 300, g)
        u = _unit(r, d)
        cols = r.choice(L, size=min(w.n_stripe_columns, L), replace=False)
        k[:, g, cols] += 3.0 * u
        q[:, g * G:(g + 1) * G] += 3.0 * u


def make_base(w: Workload):
    """Step-0 tensors in fp32 (before rounding): dict q, k, v."""
    B, Hq, Hkv, L, d = w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim
    q = _rng(w.wid, 0, _T_Q).standard_normal((B, Hq, L, d), dtype=np.float32)
    k = _rng(w.wid, 0, _T_K).standard_normal((B, Hkv, L, d), dtype=np.float32)
    v = _rng(w.wid, 0, _T_V).standard_normal((B, Hkv, L, d), dtype=np.float32)
    if w.pattern == "mix":
        _plant_mix(w, q, k)
    elif w.pattern == "columns":
        _plant_columns(w, q, k)
    if w.extra_pair_frac > 0:
        _plant_pairs(w, q, k)
    return {"q": q, "k": k, "v": v}


def _noise(w: Workload, step: int, tensor: int, shape, scale: float, out):
    n = _rng(w.wid, 1 + step, tensor).standard_normal(shape, dtype=np.float32)
    n *= np.float32(scale)
    n += out
    return n


_WALK_CHUNK = 1 << 22


def walk_nodes(total_steps: int, t: int):
    """W_t of the dyadic bridge construction as a combination of node
    tensors: a list of ((a, b), coefficient), where node (T2, T2) is the root
    (W_T2 = sqrt(T2) Z_root) and node (a, b), a < b, the midpoint draw of
    [a, b]."""
    T2 = 1
    while T2 < max(1, total_steps):
        T2 *= 2
    if not 0 <= t <= T2:
        raise ValueError(f"step {t} outside [0, {T2}]")
    wa, wb = {}, {(T2, T2): float(np.sqrt(T2))}  # W_a, W_b as {node: coefficient}
    a, b = 0, T2
    while t not in (a, b):
        c = (a + b) // 2
        wc = {k: 0.5 * v for k, v in wa.items()}
        for k, v in wb.items():
            wc[k] = wc.get(k, 0.0) + 0.5 * v
        wc[(a, b)] = wc.get((a, b), 0.0) + float(np.sqrt((b - a) / 4.0))
        if t < c:
            b, wb = c, wc
        else:
            a, wa = c, wc
    return sorted((wa if t == a else wb).items())


def _walk(w: Workload, step: int, tensor: int, x0, sigma: float):
    """x0 + sigma W_step (float32), the node draws generated and
    accumulated chunk by chunk on a thread pool (numpy releases the
    interpreter lock while filling); the result does not depend on the pool."""
    from concurrent.futures import ThreadPoolExecutor
    import os
    nodes = walk_nodes(w.total_steps, step)
    out = np.array(x0, dtype=np.float32, copy=True)
    flat = out.reshape(-1)
    n_chunks = -(-flat.size // _WALK_CHUNK)

    def fill(c):
        seg = flat[c * _WALK_CHUNK:(c + 1) * _WALK_CHUNK]
        z = np.empty(seg.size, dtype=np.float32)
        for (a, b), coef in nodes:
            _rng(w.wid, 1000 + tensor, a, b, c).standard_normal(out=z, dtype=np.float32)
            z *= np.float32(sigma * coef)
            seg += z

    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1, n_chunks))) as ex:
        list(ex.map(fill, range(n_chunks)))
    return out


def make_step(w: Workload, step: int, base=None, as_float: bool = False):
    """Inputs of denoising step `step`: dict q, k, v as stored (f32 or bf16 bits).

    With as_float=True the bf16 tensors are returned decoded to float32.
    """
    if base is None:
        base = make_base(w)
    q, k, v = base["q"], base["k"], base["v"]
    if step > 0:
        if w.step_noise == "fresh_qv":
            q = _noise(w, step, _T_Q, q.shape, w.step_sigma, q)
            v = _noise(w, step, _T_V, v.shape, w.step_sigma, v)
        elif w.step_noise == "walk":
            q = _walk(w, step, _T_Q, q, w.step_sigma)
            k = _walk(w, step, _T_K, k, w.step_sigma)
        else:
            raise ValueError(w.step_noise)
    out = {"q": q, "k": k, "v": v}
    if w.dtype == "bf16":
        out = {n: f32_to_bf16_bits(x) for n, x in out.items()}
        if as_float:
            out = {n: bf16_bits_to_f32(x) for n, x in out.items()}
    else:
        out = {n: np.ascontiguousarray(x, dtype=np.float32) for n, x in out.items()}
    return out


def tiny_random(seed: int, B, Hq, Hkv, L, d, dtype="f32", scale=1.0):
    """Plain N(0, scale^2) Q/K/V for small parity cases (no planted structure)."""
    r = _rng(9000, seed)
    q = (r.standard_normal((B, Hq, L, d)) * scale).astype(np.float32)
    k = (r.standard_normal((B, Hkv, L, d)) * scale).astype(np.float32)
    v = r.standard_normal((B, Hkv, L, d)).astype(np.float32)
    out = {"q": q, "k": k, "v": v}
    if dtype == "bf16":
        out = {n: f32_to_bf16_bits(x) for n, x in out.items()}
    return out


def score_jump(seed: int, B, Hq, Hkv, L, d, jump, n_low=64, dtype="bf16"):
    """Q near +1 in every component; the first n_low keys near -jump, every
    37th later key near +jump and the rest small, so the first keys score
    about 2 jump sqrt(d) below the largest ones.  V is N(0, 1/4)."""
    r = _rng(9100, seed)
    q = (1.0 + 0.1 * r.standard_normal((B, Hq, L, d))).astype(np.float32)
    k = (0.3 * r.standard_normal((B, Hkv, L, d))).astype(np.float32)
    k[:, :, :n_low] = -jump * (1.0 + 0.1 * r.standard_normal((B, Hkv, min(n_low, L), d)))
    hi = np.arange(n_low, L, 37)
    k[:, :, hi] = jump * (1.0 + 0.1 * r.standard_normal((B, Hkv, len(hi), d)))
    v = (0.5 * r.standard_normal((B, Hkv, L, d))).astype(np.float32)
    out = {"q": q, "k": k, "v": v}
    if dtype == "bf16":
        out = {n: f32_to_bf16_bits(x) for n, x in out.items()}
    return out


_T_KC, _T_VC = 3, 4


def make_losa_base(w: LosaWorkload):
    """Prefix caches and iteration-0 block tensors in fp32: dict k_cache,
    v_cache, q, k_blk, v_blk."""
    B, Hq, Hkv, Lp, Bs, d = w.batch, w.q_heads, w.kv_heads, w.prefix_len, w.block_len, w.head_dim
    G = Hq // Hkv
    kc = _rng(w.wid, 0, _T_KC).standard_normal((B, Hkv, Lp, d), dtype=np.float32)
    vc = _rng(w.wid, 0, _T_VC).standard_normal((B, Hkv, Lp, d), dtype=np.float32)
    q = _rng(w.wid, 0, _T_Q).standard_normal((B, Hq, Bs, d), dtype=np.float32)
    kb = _rng(w.wid, 0, _T_K).standard_normal((B, Hkv, Bs, d), dtype=np.float32)
    vb = _rng(w.wid, 0, _T_V).standard_normal((B, Hkv, Bs, d), dtype=np.float32)
    n_units = -(-Lp // UNIT)
    n_pages = Lp // w.page
    for g in range(Hkv):
        r = _rng(w.wid, 400, g)
        qs = slice(g * G, (g + 1) * G)
        kind = g % 4
        u = _unit(r, d)
        if kind == 0:
            kc[:, g, :min(UNIT, Lp)] += 3.0 * u
            q[:, qs] += 3.0 * u
        elif kind == 1:
            kc[:, g, max(0, Lp - 4 * UNIT):] += 3.0 * u
            q[:, qs] += 3.0 * u
        elif kind == 2:
            for c in r.choice(n_units, size=min(4, n_units), replace=False):
                kc[:, g, c * UNIT:min(Lp, (c + 1) * UNIT)] += 3.0 * u
            q[:, qs] += 3.0 * u
        for i in range(Bs):
            wi = _unit(r, d)
            q[:, qs, i] += 2.0 * wi
            for P in r.choice(n_pages, size=min(w.pages_per_token, n_pages), replace=False):
                kc[:, g, P * w.page:(P + 1) * w.page] += 2.0 * wi
    return {"k_cache": kc, "v_cache": vc, "q": q, "k_blk": kb, "v_blk": vb}


def _losa_rounded(w: LosaWorkload, x):
    return f32_to_bf16_bits(x) if w.dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def make_losa_cache(w: LosaWorkload, base=None):
    """The prefix caches as stored: dict k_cache, v_cache."""
    base = make_losa_base(w) if base is None else base
    return {n: _losa_rounded(w, base[n]) for n in ("k_cache", "v_cache")}


def make_losa_iteration(w: LosaWorkload, t: int, base=None):
    """The block's q, k_blk, v_blk at iteration t, as stored."""
    base = make_losa_base(w) if base is None else base
    x = {n: base[n].copy() for n in ("q", "k_blk", "v_blk")}
    Bs = w.block_len
    for s in range(1, t + 1):
        pick = _rng(w.wid, 1 + s, 9).choice(Bs, size=min(w.n_moving, Bs), replace=False)
        sig = np.full(Bs, w.sigma_still, dtype=np.float32)
        sig[pick] = w.sigma_move
        for ti, n in enumerate(("q", "k_blk", "v_blk")):
            noise = _rng(w.wid, 1 + s, 10 + ti).standard_normal(x[n].shape, dtype=np.float32)
            x[n] += noise * sig[None, None, :, None]
    return {n: _losa_rounded(w, a) for n, a in x.items()}
