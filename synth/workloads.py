"""Shapes of the BDLM attention workloads.

The paper (Block Parallelism For Efficient Distributed Long-Context Diffusion
Language Model Training) trains at 64K-512K context with block sizes 128-1024
(its App. K robustness study) and shards the clean sequence over 16 ranks at
256K (its Table 1 setting).  These workloads take those shapes on synthetic
data; none of them comes from a dataset.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int            # L: clean tokens (= corrupted tokens)
    block: int             # B
    hq: int
    hkv: int
    head_dim: int
    dtype: str             # "f32" or "bf16"
    seed: int
    q_std: float           # std of Q/K/V draws (before the dtype cast)
    outlier_frac: float = 0.0   # fraction of key rows scaled by outlier_mult
    outlier_mult: float = 8.0
    # CSBP share mode (one rank's corrupted blocks against a streamed clean prefix)
    share_blocks: int = 0       # number of local corrupted blocks (0 = full mode)
    share_chunk: int = 0        # clean tokens per streamed chunk
    clean_share: bool = False   # also the rank's own clean query shard (context-parallel half)
    share_ranks: int = 16       # ranks the clean sequence is sharded over
    units: int = 64             # sampled (batch, stream, block, head) units for the oracle
    note: str = ""

    @property
    def nblocks(self) -> int:
        return self.seqlen // self.block

    @property
    def scale(self) -> float:
        return 1.0 / (self.head_dim ** 0.5)

    def with_block(self, block: int, seed: Optional[int] = None) -> "Workload":
        d = dict(self.__dict__)
        d["block"] = block
        d["name"] = f"{self.name.split('_B')[0]}_B{block}"
        if seed is not None:
            d["seed"] = seed
        return Workload(**d)


def _w(**kw) -> Workload:
    return Workload(**kw)


WORKLOADS = {
    # Tiny fp32 case: the full oracle finishes in well under a second.
    "tiny_f32": _w(name="tiny_f32", batch=1, seqlen=256, block=16, hq=2, hkv=2,
                   head_dim=64, dtype="f32", seed=1, q_std=1.0 / 8.0),
    # bf16, MHA, short context.
    "mha_8k": _w(name="mha_8k", batch=2, seqlen=4096, block=32, hq=16, hkv=16,
                 head_dim=128, dtype="bf16", seed=2, q_std=1.0 / 128 ** 0.5),
    # Headline: 2L = 64K tokens, GQA 32/8, 1 % outlier key rows x8.
    "gqa_64k": _w(name="gqa_64k", batch=1, seqlen=32768, block=64, hq=32, hkv=8,
                  head_dim=128, dtype="bf16", seed=3, q_std=1.0 / 128 ** 0.5,
                  outlier_frac=0.01),
    # One rank's CSBP share at 256K: 16 corrupted blocks of 1024 at seeded
    # positions, clean prefix streamed in 8192-token chunks.
    "csbp_share_256k": _w(name="csbp_share_256k", batch=1, seqlen=262144, block=1024,
                          hq=32, hkv=8, head_dim=128, dtype="bf16", seed=4,
                          q_std=1.0 / 128 ** 0.5, share_blocks=16, share_chunk=8192),
    # The whole attention share of one of 16 ranks at 256K: the corrupted blocks
    # above plus the rank's zigzag shard of the clean sequence (16 clean blocks
    # of 1024, query side), both against the streamed clean K/V.
    "csbp_rank_256k": _w(name="csbp_rank_256k", batch=1, seqlen=262144, block=1024,
                         hq=32, hkv=8, head_dim=128, dtype="bf16", seed=4,
                         q_std=1.0 / 128 ** 0.5, share_blocks=16, share_chunk=8192,
                         clean_share=True, share_ranks=16),
    # Block-size sweep at 2L = 256K.
    "sweep_256k_B128": _w(name="sweep_256k_B128", batch=1, seqlen=131072, block=128, hq=32,
                          hkv=8, head_dim=128, dtype="bf16", seed=5128,
                          q_std=1.0 / 128 ** 0.5),
    "sweep_256k_B256": _w(name="sweep_256k_B256", batch=1, seqlen=131072, block=256, hq=32,
                          hkv=8, head_dim=128, dtype="bf16", seed=5256,
                          q_std=1.0 / 128 ** 0.5),
    "sweep_256k_B512": _w(name="sweep_256k_B512", batch=1, seqlen=131072, block=512, hq=32,
                          hkv=8, head_dim=128, dtype="bf16", seed=5512,
                          q_std=1.0 / 128 ** 0.5),
    "sweep_256k_B1024": _w(name="sweep_256k_B1024", batch=1, seqlen=131072, block=1024, hq=32,
                           hkv=8, head_dim=128, dtype="bf16", seed=6024,
                           q_std=1.0 / 128 ** 0.5),
}

