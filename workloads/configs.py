"""The five attention workloads, as plain parameters.

Each workload is named by what it is and its sizes.  The step schedule is
given as explicit integers (warm-up length, selection step, refresh interval or
list), so that nothing here computes part of the method.

Sources of the shapes and schedules:
  * SparseD (Sparse Attention for Diffusion Language Models), abstract: full
    attention for the early steps, a head-specific pattern computed once and
    reused; the 64k-context, 1,024-step operating point.
  * Step-dLLM (arXiv 2611.01320), abstract: block-sparse mask refreshed at
    anchor steps with a head-adaptive global budget; LLaDA-1.5 at 8K context,
    256 steps, 90% sparsity.
  * PulseCol (arXiv 2605.20813), abstract: column-sparse pattern found at an
    early step and refreshed at a few intermediate steps.
  * LoSA (Locality Aware Sparse Attention for block-wise diffusion LMs),
    sections 3 and 5: a block denoised on top of a cached prefix, a few Active
    tokens per iteration, a per-query budget of 128 prefix tokens; Trado-8B /
    SDAR-8B shaped heads (32 query heads, 8 kv heads, d = 128).
"""

from dataclasses import dataclass
from typing import Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                      # seed namespace of the generator
    batch: int
    q_heads: int
    kv_heads: int
    seq_len: int
    head_dim: int
    dtype: str                    # "f32" or "bf16"
    block: int                    # block_q == block_k
    # step schedule (explicit integers)
    total_steps: int
    dense_steps: int
    select_step: int
    refresh_interval: int = 0     # 0: no periodic refresh
    refresh_steps: Tuple[int, ...] = ()
    refresh_dense: bool = False
    selector: str = "blocks"      # "blocks" (pooled), "blocks_exact" (exact block mass) or "columns"
    # budget
    budget: str = "topk"          # "topk" or "mass"
    keep_frac: float = 0.0        # top-k fraction of key blocks per row
    mass: float = 0.0             # cumulative pooled-mass target
    max_mean_density: float = 1.0  # global cap on the mean kept fraction
    column_keep_frac: float = 0.0  # top fraction of key columns per kv head
    # adaptive anchors (blocks): probe every probe_interval sparse steps and
    # adopt the probe when its overlap with the cached pattern is below min_overlap
    probe_interval: int = 0
    min_overlap: float = 0.0
    # generator
    pattern: str = "mix"          # "mix" (round-robin head types) or "columns"
    extra_pair_frac: float = 0.0  # fraction of (I, J) block pairs given extra alignment
    n_stripe_columns: int = 0     # single-token stripes per kv head ("columns")
    step_noise: str = "walk"      # "fresh_qv" or "walk"
    step_sigma: float = 0.02
    notes: str = ""

    @property
    def n_blocks(self) -> int:
        return -(-self.seq_len // self.block)


WORKLOADS = {
    w.name: w
    for w in [
        Workload(
            name="tiny_fp32_h4_l512", wid=1, batch=1, q_heads=4, kv_heads=4,
            seq_len=512, head_dim=64, dtype="f32", block=64,
            total_steps=4, dense_steps=1, select_step=0,
            budget="topk", keep_frac=0.25,
            step_noise="fresh_qv", step_sigma=0.05,
            notes="tiny single layer; step 0 dense + top-25% block mask, steps 1-3 reuse it",
        ),
        Workload(
            name="llada8b_8k", wid=2, batch=1, q_heads=32, kv_heads=32,
            seq_len=8192, head_dim=128, dtype="bf16", block=64,
            total_steps=256, dense_steps=1, select_step=0, refresh_interval=32,
            budget="mass", mass=0.95, max_mean_density=0.10,
            step_noise="walk", step_sigma=0.02,
            notes="head-adaptive mass budget (95% pooled mass, mean density <= 10%), refresh every 32 steps",
        ),
        Workload(
            name="sparsed_32k", wid=3, batch=1, q_heads=32, kv_heads=32,
            seq_len=32768, head_dim=128, dtype="bf16", block=128,
            total_steps=128, dense_steps=26, select_step=26,
            budget="topk", keep_frac=0.10, extra_pair_frac=0.02,
            step_noise="walk", step_sigma=0.02,
            notes="dense for the first 20% of 128 steps, then a fixed top-10% block mask",
        ),
        Workload(
            name="sparsed_64k", wid=4, batch=1, q_heads=32, kv_heads=32,
            seq_len=65536, head_dim=128, dtype="bf16", block=128,
            total_steps=1024, dense_steps=205, select_step=205,
            budget="topk", keep_frac=0.05,
            step_noise="walk", step_sigma=0.02,
            notes="dense for steps 0-204, then a fixed top-5% block mask for 819 steps",
        ),
        Workload(
            name="pulsecol_dream7b_16k", wid=5, batch=1, q_heads=28, kv_heads=4,
            seq_len=16384, head_dim=128, dtype="bf16", block=64,
            total_steps=192, dense_steps=1, select_step=0,
            refresh_steps=(64, 128), refresh_dense=True, selector="columns",
            column_keep_frac=0.03, pattern="columns", n_stripe_columns=512,
            step_noise="walk", step_sigma=0.02,
            notes="GQA 28/4; top-3% key columns per kv head, refreshed at 64 and 128",
        ),
    ]
}


@dataclass(frozen=True)
class LosaWorkload:
    """A block of block_len tokens denoised on top of a cached prefix of
    prefix_len tokens: iteration 0 dense, iterations 1..steps_per_block-1
    LoSA-style (n_active Active tokens, pages_per_query pages of `page`
    tokens kept per Active query)."""
    name: str
    wid: int
    batch: int
    q_heads: int
    kv_heads: int
    prefix_len: int
    block_len: int
    head_dim: int
    dtype: str
    page: int
    pages_per_query: int
    n_active: int
    steps_per_block: int
    # generator: per iteration, n_moving tokens of the block change by
    # sigma_move * N(0, 1), the others by sigma_still * N(0, 1)
    n_moving: int = 6
    sigma_move: float = 0.5
    sigma_still: float = 0.01
    pages_per_token: int = 2      # prefix pages aligned with each block token
    notes: str = ""


LOSA_WORKLOADS = {
    w.name: w
    for w in [
        LosaWorkload(
            name="losa_sdar8b_32k", wid=6, batch=1, q_heads=32, kv_heads=8, prefix_len=32768,
            block_len=32, head_dim=128, dtype="bf16", page=16, pages_per_query=8, n_active=8,
            steps_per_block=8,
            notes="32-token block over a 32K cached prefix; 8 Active tokens, 8 pages of 16 (128 tokens) per query",
        ),
    ]
}


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError as e:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from e


def scaled(w, **overrides):
    """A copy of a workload with some fields replaced (smaller parity shapes)."""
    d = dict(w.__dict__)
    d.update(overrides)
    return type(w)(**d)
