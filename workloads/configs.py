"""The decode workloads, as plain parameters.

Shapes follow the pages' statement of the problem: L layers, H_kv key/value
heads, head dimension d, block size B, b bytes per stored scalar ("Serving
Language Models Within a Memory Budget", section 3 and eq. (1); "PagedAttention
and Online Inference", core eq. (1)).  The five lengths 37/91/128/201/511 are
the worked example of "PagedAttention and Online Inference" (section 2 and the
recalculable worked example).  The OPT-13B shape (40 heads x 128 dims x 40
layers, FP16) is the per-token cache example of the NetLeverage article
"vLLM PagedAttention and continuous batching" (section "Why it matters").

Lengths are context lengths *including* the token appended by the decode
step being computed.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

FIVE_LENGTHS: Tuple[int, ...] = (37, 91, 128, 201, 511)


@dataclass(frozen=True)
class DecodeConfig:
    cfg_id: int
    name: str
    L: int                  # layers
    Hq: int                 # query heads
    Hkv: int                # key/value heads
    d: int                  # head dimension
    B: int                  # block size (token slots per block)
    dtype: str              # "f16" or "bf16" (Q, K, V and output storage)
    length_kind: str        # "five", "uniform", "fixed", "lognormal_branches"
    S: int                  # sequences in the decode batch
    pool_kind: str          # "fixed", "scaled", "exact", "branch_bound"
    pool_blocks: Optional[int] = None   # for pool_kind == "fixed"
    pool_scale: float = 1.0             # for pool_kind == "scaled"
    uniform_lo: int = 0
    uniform_hi: int = 0
    fixed_len: int = 0
    prompts: int = 0                    # lognormal_branches: number of prompts
    branches: int = 0                   # lognormal_branches: samples per prompt
    lognormal_median: float = 0.0
    lognormal_sigma: float = 0.0
    max_len: int = 0
    steps: int = 1                      # decode steps the workload runs
    share_prefix_tokens: int = 0        # cfg2: tokens of seq 0 mapped by seqs 1..S-1
    beam: bool = False                  # lognormal_branches: reselect the branches every step
    description: str = field(default="", compare=False)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def elem_bytes(self) -> int:
        return 2


CONFIGS = {
    1: DecodeConfig(
        cfg_id=1, name="five_lengths_b16_gqa4_f16",
        L=1, Hq=8, Hkv=2, d=128, B=16, dtype="f16",
        length_kind="five", S=5, pool_kind="fixed", pool_blocks=64,
        description="one layer, one decode step, lengths 37/91/128/201/511, "
                    "B=16, 8 query / 2 KV heads, d=128, fp16, 64-block pool"),
    2: DecodeConfig(
        cfg_id=2, name="five_lengths_b32_prefix_share_f16",
        L=1, Hq=8, Hkv=2, d=128, B=32, dtype="f16",
        length_kind="five", S=5, pool_kind="fixed", pool_blocks=64,
        share_prefix_tokens=64,
        description="config 1 at B=32; sequences 2-4 map the first two physical "
                    "blocks of sequence 1 (refcount 4); sequence 1's write lands "
                    "in the shared partial block and triggers copy-on-write"),
    3: DecodeConfig(
        cfg_id=3, name="gqa32x8_d128_bf16_b16_s64",
        L=32, Hq=32, Hkv=8, d=128, B=16, dtype="bf16",
        length_kind="uniform", S=64, uniform_lo=512, uniform_hi=4096,
        pool_kind="scaled", pool_scale=1.25,
        description="GQA decode, 32 layers, 32 query / 8 KV heads, d=128, bf16, "
                    "batch 64, lengths uniform in [512,4096], B=16, pool 1.25x "
                    "used blocks, shuffled physical blocks"),
    4: DecodeConfig(
        cfg_id=4, name="mha32_d128_f16_b32_s32_ctx4096",
        L=32, Hq=32, Hkv=32, d=128, B=32, dtype="f16",
        length_kind="fixed", S=32, fixed_len=4096, pool_kind="exact",
        description="MHA decode, 32 heads, d=128, fp16, batch 32 at context "
                    "4096, B=32, one layer per launch over 32 layers"),
    5: DecodeConfig(
        cfg_id=5, name="opt13b_shape_mha40_f16_b16_4branch",
        L=40, Hq=40, Hkv=40, d=128, B=16, dtype="f16",
        length_kind="lognormal_branches", S=256, prompts=64, branches=4,
        lognormal_median=300.0, lognormal_sigma=0.8, max_len=2048, steps=32,
        pool_kind="branch_bound",
        description="OPT-13B-shaped decode: 40 heads x 128 x 40 layers, fp16, "
                    "64 prompts x 4 sampled branches sharing prompt blocks, "
                    "log-normal prompt lengths (median 300, max 2048), B=16, "
                    "32 decode steps with copy-on-write"),
    6: DecodeConfig(
        cfg_id=6, name="opt13b_shape_mha40_f16_b16_beam4",
        L=40, Hq=40, Hkv=40, d=128, B=16, dtype="f16",
        length_kind="lognormal_branches", S=256, prompts=64, branches=4,
        lognormal_median=300.0, lognormal_sigma=0.8, max_len=2048, steps=32,
        pool_kind="branch_bound", beam=True,
        description="beam search of width 4 over config 5's shape: before every "
                    "step each prompt's 4 beams are reselected from its current "
                    "beams (seeded parents, better beams more likely), dropped "
                    "beams release their blocks, shared last blocks are copied "
                    "on write"),
}


def get_config(cfg_id: int) -> DecodeConfig:
    return CONFIGS[int(cfg_id)]
