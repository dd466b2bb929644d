"""The five workloads of the CSA / HCA / DSA hot path, by name and size.

Shapes follow the Hugging Face Transformers model pages: "DeepSeek-V4"
(DeepseekV4Config: head_dim 512, 64 heads, one K=V head, sliding_window 128,
index_n_heads 64, index_head_dim 128, index_topk 512, compress_rates CSA 4 /
HCA 128, compress_rope_theta 160000) and "DeepSeek-V3.2" (DeepseekV32Config:
index_topk 2048, 128 heads, kv_lora_rank 512 + qk_rope_head_dim 64, rope_theta
10000).  Inputs are synthetic (seeded normal draws); no checkpoint is used.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "csa" | "hca" | "dsa"
    dtype: str           # "f32" | "bf16"
    B: int               # sequences
    S: int               # query rows per sequence
    H: int               # query heads
    D: int               # K=V row width (head_dim)
    dv: int              # output width: D, or D - rope_dim (DSA latent)
    rope_dim: int        # trailing rotated channels
    m: int               # compression rate (1 = token level)
    overlap: int         # 1 = windows of 2m (CSA), 0 = m (HCA, DSA)
    ctx: int             # tokens the pool covers: T = ctx // m
    n_idx_heads: int     # indexer heads (0 = no indexer)
    idx_dim: int         # indexer head dim
    topk: int            # index_topk (0 = dense over ready entries)
    window: int          # sliding_window
    theta: float
    act_scale: float     # activations ~ act_scale * N(0, 1)
    sink: bool
    q_pos0: int = 0      # absolute position of query row 0
    decode: bool = False  # caches given directly (pool, index keys, window)

    @property
    def T(self) -> int:
        return self.ctx // self.m

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def rows(self) -> int:
        return self.B * self.S

    @property
    def n_pos(self) -> int:
        """RoPE table length covering every position used (queries; and the
        tokens and entries the compressor rotates when caches are built here)."""
        if self.decode:
            return self.q_pos0 + self.S
        return max(self.q_pos0 + self.S, self.ctx)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # Tiny CSA, fp32, B=1, S=256, 4 heads, head_dim 64, rope 16, m=4 overlapping
    # -> 64 entries; indexer 2 heads x 32, top-16, window 32; N(0,1), seed 0.
    "tiny_csa_f32": Workload("tiny_csa_f32", "csa", "f32", B=1, S=256, H=4, D=64, dv=64,
                             rope_dim=16, m=4, overlap=1, ctx=256, n_idx_heads=2,
                             idx_dim=32, topk=16, window=32, theta=160000.0,
                             act_scale=1.0, sink=True),
    # CSA prefill, bf16, S=8192, 64 heads x 512, rope 64, m=4 -> 2048 entries;
    # indexer 64 x 128, top-512, window 128; activations 0.5*N(0,1).
    "csa_prefill_bf16": Workload("csa_prefill_bf16", "csa", "bf16", B=1, S=8192, H=64,
                                 D=512, dv=512, rope_dim=64, m=4, overlap=1, ctx=8192,
                                 n_idx_heads=64, idx_dim=128, topk=512, window=128,
                                 theta=160000.0, act_scale=0.5, sink=True),
    # HCA layer, bf16, S=65536, m'=128 non-overlapping -> 512 entries, dense over
    # ready entries plus window 128; N(0,1); per-head sink.
    "hca_bf16": Workload("hca_bf16", "hca", "bf16", B=1, S=65536, H=64, D=512, dv=512,
                         rope_dim=64, m=128, overlap=0, ctx=65536, n_idx_heads=0,
                         idx_dim=0, topk=0, window=128, theta=160000.0, act_scale=1.0,
                         sink=True),
    # CSA decode, bf16, 64 sequences x 1 new token after 131072 cached tokens
    # (32768 entries at m=4); top-2048, window 128; caches N(0,1).
    "csa_decode_bf16": Workload("csa_decode_bf16", "csa", "bf16", B=64, S=1, H=64, D=512,
                                dv=512, rope_dim=64, m=4, overlap=1, ctx=131072,
                                n_idx_heads=64, idx_dim=128, topk=2048, window=128,
                                theta=160000.0, act_scale=1.0, sink=True, q_pos0=131072,
                                decode=True),
    # DSA token-level indexer (m=1), bf16, S=32768, indexer 64 x 128, top-2048
    # tokens; sparse MQA with 128 heads, head_dim 576 (rope 64), latent 512 as
    # value; no window, no sink.
    "dsa_bf16": Workload("dsa_bf16", "dsa", "bf16", B=1, S=32768, H=128, D=576, dv=512,
                         rope_dim=64, m=1, overlap=0, ctx=32768, n_idx_heads=64,
                         idx_dim=128, topk=2048, window=0, theta=10000.0, act_scale=1.0,
                         sink=False),
}
