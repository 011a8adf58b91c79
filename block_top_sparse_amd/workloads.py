"""Workload shapes for block top-k sparse decode attention.

The shapes stand in for the decode workloads the Kinetics pages measure
(rebuttal page "Kinetics: Rethinking Test-Time Scaling Law", "W2 & Q2:
Real-world latency benchmarks": Qwen3 decode against a 32K-token KV cache,
Best-of-N batches; answer Q4: budgets of 1024 tokens as (block, top-k) =
(16,64), (32,32), (64,16)).  Head layouts follow the Qwen3 8B / 14B / 32B
attention shapes (32/8, 40/8, 64/8 query/KV heads, head_dim 128).

No arithmetic of the method lives here: only sizes, seeds and byte counts
used to report bandwidth.
"""
from dataclasses import dataclass, field, replace
from typing import List


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    hq: int
    hkv: int
    ctx_len: int
    block: int
    topk: int
    dtype: str            # "f32" or "bf16"
    seed: int
    head_dim: int = 128
    heavy_blocks: int = 0  # blocks per pair whose keys are pushed toward q
    t_cap: int = 0         # cache capacity in tokens (0: equal to ctx_len)
    share_n: int = 0       # samples per shared prompt (0: no shared prompt)
    prompt_len: int = 0    # tokens of each shared prompt
    quest: bool = False    # Quest-style representative (minimum and maximum rows)
    page_size: int = 0     # paged K/V (tokens per page; 0: contiguous caches)
    len_std: int = 0       # per-sequence lengths ~ N(ctx_len - 3 len_std, len_std), clipped

    @property
    def gqa(self) -> int:
        return self.hq // self.hkv

    @property
    def cap(self) -> int:
        return self.t_cap or self.ctx_len

    @property
    def nb(self) -> int:
        return (self.ctx_len + self.block - 1) // self.block

    @property
    def nb_cap(self) -> int:
        return (self.cap + self.block - 1) // self.block

    @property
    def esize(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def pairs(self) -> int:
        return self.batch * self.hkv

    @property
    def k_eff(self) -> int:
        return min(self.topk, self.nb)

    # ---- algorithmic bytes (what the method has to move, per call) ----
    def bytes_summary_scan(self) -> int:
        """The summary rows a step must read to rank the blocks: none when
        every block is kept (the scores cannot change the selection, and the
        step without a scores output skips them)."""
        if self.k_eff >= self.nb:
            return 0
        if self.quest:  # two summary rows per block
            return 2 * self.pairs * self.nb * self.head_dim * self.esize
        if self.share_n:
            # a prompt's block summaries are read once for its n_share samples
            pb = self.prompt_len // self.block
            units = self.pairs // self.share_n
            return (units * pb + self.pairs * (self.nb - pb)) * self.head_dim * self.esize
        return self.pairs * self.nb * self.head_dim * self.esize

    def kept_tokens(self) -> int:
        """Tokens of the kept blocks that lie inside the context, per pair
        (the blocks are the top k; for the byte model take the last block as
        partial only when it must be kept, i.e. when every block is kept)."""
        if self.k_eff >= self.nb:
            return self.ctx_len
        return self.k_eff * self.block

    def bytes_gather(self) -> int:
        return self.pairs * self.kept_tokens() * self.head_dim * self.esize * 2

    def bytes_q_out(self) -> int:
        return self.batch * self.hq * self.head_dim * self.esize * 2

    def bytes_update(self) -> int:
        """Newest-block summary update of one decode step: read the newest
        block's keys (at most one block) and write one summary row.  None
        with blocks of one token (the keys are the summaries)."""
        if self.block == 1:
            return 0
        if self.quest:  # the newest block's keys in, its two rows out
            newest = self.ctx_len - (self.nb - 1) * self.block
            return self.pairs * (newest + 2) * self.head_dim * self.esize
        newest = self.ctx_len - (self.nb - 1) * self.block
        return self.pairs * (newest + 1) * self.head_dim * self.esize

    def bytes_sparse_step(self) -> int:
        return (self.bytes_summary_scan() + self.bytes_gather() + self.bytes_q_out()
                + self.bytes_update())

    def bytes_dense(self) -> int:
        return (self.pairs * self.ctx_len * self.head_dim * self.esize * 2
                + self.bytes_q_out())

    def cache_bytes(self) -> int:
        return 2 * self.pairs * self.cap * self.head_dim * self.esize

    def summary_bytes(self) -> int:
        return self.pairs * self.nb_cap * self.head_dim * self.esize

    def describe(self) -> dict:
        return {"workload": self.name, "batch": self.batch, "hq": self.hq, "hkv": self.hkv,
                "head_dim": self.head_dim, "ctx_len": self.ctx_len, "block": self.block,
                "topk_blocks": self.topk, "budget_tokens": self.topk * self.block,
                "dtype": self.dtype, "heavy_blocks": self.heavy_blocks, "seed": self.seed}

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


TINY = Workload("tiny-gqa4-ctx4096-f32", batch=1, hq=8, hkv=2, ctx_len=4096, block=16, topk=32,
                dtype="f32", seed=1001)
QWEN3_8B = Workload("qwen3-8b-longcot-b32-ctx32k", batch=32, hq=32, hkv=8, ctx_len=32768,
                    block=16, topk=64, dtype="bf16", seed=1002)
QWEN3_14B = Workload("qwen3-14b-b64-ctx32k-heavy", batch=64, hq=40, hkv=8, ctx_len=32768,
                     block=32, topk=64, dtype="bf16", seed=1003, heavy_blocks=4)
QWEN3_32B = Workload("qwen3-32b-b32-ctx64k", batch=32, hq=64, hkv=8, ctx_len=65536, block=64,
                     topk=64, dtype="bf16", seed=1004)

MAIN = [TINY, QWEN3_8B, QWEN3_14B, QWEN3_32B]

# Variable lengths in a paged cache: the qwen3-8b layer with lengths of mean
# 32K and standard deviation 2K (rebuttal, Q3 "Diverse prompt lengths"),
# ctx_len the bound, 256-token pages in a shuffled pool.
PAGED = [
    Workload("paged-qwen3-8b-b32-ctx32k-sd2k", batch=32, hq=32, hkv=8, ctx_len=32768 + 6144,
             block=16, topk=64, dtype="bf16", seed=1402, page_size=256, len_std=2048),
]

# Quest-style representative on the qwen3-8b decode layer.
QUEST = [
    Workload("quest-qwen3-8b-b32-ctx32k", batch=32, hq=32, hkv=8, ctx_len=32768, block=16,
             topk=64, dtype="bf16", seed=1302, quest=True),
]

# Shared-prompt Best-of-N: 4 prompts x 8 samples on the qwen3-8b layer, a
# 16K-token prompt common to each prompt's samples, 16K tokens of their own.
SHARED = [
    Workload("bon-qwen3-8b-n8-prompt16k-ctx32k", batch=32, hq=32, hkv=8, ctx_len=32768,
             block=16, topk=64, dtype="bf16", seed=1202, share_n=8, prompt_len=16384),
]

# Token-level top-k (block 1): the headline decode shape with a budget of
# 1024 tokens, and a long-context Best-of-8 shape.
TOKEN = [
    Workload("tok-qwen3-8b-b32-ctx32k-budget1024", batch=32, hq=32, hkv=8, ctx_len=32768,
             block=1, topk=1024, dtype="bf16", seed=1102),
    Workload("tok-qwen3-32b-b8-ctx128k-budget4096", batch=8, hq=64, hkv=8, ctx_len=131072,
             block=1, topk=4096, dtype="bf16", seed=1104),
]

SWEEP_BATCH = (8, 32, 128)
SWEEP_CTX = (8192, 32768, 131072)
SWEEP_BLOCK = (16, 32, 64)
SWEEP_BUDGET = (256, 1024, 4096, 8192)


def sweep() -> List[Workload]:
    """Budget / length sweep on the Qwen3-32B head layout (64q/8kv, d=128,
    bf16): every (batch, ctx, block, token budget) point in row-major order,
    then the keep-every-block (dense-equivalent) point of each
    (batch, ctx, block)."""
    pts = []
    p = 0
    for b in SWEEP_BATCH:
        for L in SWEEP_CTX:
            for B in SWEEP_BLOCK:
                for budget in SWEEP_BUDGET:
                    pts.append(Workload(f"sweep-b{b}-ctx{L}-blk{B}-budget{budget}", batch=b, hq=64,
                                        hkv=8, ctx_len=L, block=B, topk=budget // B,
                                        dtype="bf16", seed=5000 + p))
                    p += 1
    for b in SWEEP_BATCH:
        for L in SWEEP_CTX:
            for B in SWEEP_BLOCK:
                pts.append(Workload(f"sweep-b{b}-ctx{L}-blk{B}-allblocks", batch=b, hq=64, hkv=8,
                                    ctx_len=L, block=B, topk=L // B, dtype="bf16", seed=5000 + p))
                p += 1
    return pts


def by_name(name: str) -> Workload:
    for w in MAIN + TOKEN + SHARED + QUEST + PAGED + sweep():
        if w.name == name:
            return w
    raise KeyError(name)
