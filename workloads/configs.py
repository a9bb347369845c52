"""The five workload shapes the hybrid prefill is exercised and measured on.

Each entry fixes the tensor shapes, the value distributions, the router's
widths and init, the sparse-attention geometry (64-token blocks, sink blocks,
retained fraction) and how many KV heads per sequence are meant to route to
sparse attention.  The shapes follow the backbones the pages evaluate on
(Elastic Attention paper body: the backbone paragraph names Qwen3-4B/8B and
Llama-3.1-8B; the RULER paragraph evaluates 8K-256K contexts; the training
paragraph uses 8K-64K sequences).  Sizes are in tokens.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                       # "f32" or "bf16": the element type of Q, K, V, O
    seq_lens: tuple | None           # fixed sequence lengths, or None: drawn (varlen)
    n_seqs: int
    Hq: int
    Hkv: int
    d: int
    q_std: float = 1.0
    k_std: float = 1.0
    v_std: float = 1.0
    lowrank: int = 0                 # rank of an extra seeded low-rank term in K (0 = none)
    task_hidden: int = 512
    router_hidden: int = 64
    w_std: float = 0.05              # N(0, w_std) for every router weight and bias
    pool_len: int = 100
    block: int = 64
    n_sink: int = 1                  # attention-sink blocks kept by sparse heads
    keep_fraction: float = 0.2       # retained share of key blocks for sparse heads
    sa_heads: tuple | None = None    # per sequence, number of KV heads routed to SA; None = natural
    start_seed: int = 1
    varlen_range: tuple = (4096, 65536)
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


WORKLOADS = {
    w.name: w
    for w in [
        Workload(
            name="tiny_f32_s512", dtype="f32", seq_lens=(512,), n_seqs=1, Hq=4, Hkv=2, d=64,
            task_hidden=256, router_hidden=32, w_std=0.05, n_sink=1, keep_fraction=0.2,
            sa_heads=None, start_seed=1,
            notes="fp32 correctness case; natural routing, margin-checked",
        ),
        Workload(
            name="llama8b_s32k", dtype="bf16", seq_lens=(32768,), n_seqs=1, Hq=32, Hkv=8, d=128,
            k_std=0.5, task_hidden=1024, router_hidden=64, w_std=0.02, n_sink=2,
            keep_fraction=0.2, sa_heads=(4,), start_seed=2,
            notes="Llama-3.1-8B-shaped layer; router of 271,682 parameters",
        ),
        Workload(
            name="qwen4b_s128k_sa2", dtype="bf16", seq_lens=(131072,), n_seqs=1, Hq=32, Hkv=8,
            d=128, task_hidden=512, router_hidden=64, w_std=0.05, n_sink=1, keep_fraction=0.2,
            sa_heads=(2,), start_seed=3,
            notes="Qwen3-4B-shaped layer at 128K, 2 of 8 KV heads sparse",
        ),
        Workload(
            name="qwen4b_s128k_sa6", dtype="bf16", seq_lens=(131072,), n_seqs=1, Hq=32, Hkv=8,
            d=128, task_hidden=512, router_hidden=64, w_std=0.05, n_sink=1, keep_fraction=0.2,
            sa_heads=(6,), start_seed=3,
            notes="Qwen3-4B-shaped layer at 128K, 6 of 8 KV heads sparse",
        ),
        Workload(
            name="extrap_s256k", dtype="bf16", seq_lens=(262144,), n_seqs=1, Hq=32, Hkv=8, d=128,
            lowrank=8, task_hidden=512, router_hidden=64, w_std=0.05, n_sink=4,
            keep_fraction=0.1, sa_heads=(6,), start_seed=4,
            notes="length-extrapolation layer at 256K with a rank-8 term in K",
        ),
        Workload(
            name="varlen8", dtype="bf16", seq_lens=None, n_seqs=8, Hq=32, Hkv=8, d=128,
            task_hidden=512, router_hidden=64, w_std=0.05, n_sink=1, keep_fraction=0.2,
            sa_heads=(0, 1, 2, 3, 5, 6, 7, 8), start_seed=5,
            notes="8 sequences, lengths log-uniform in [4096, 65536]; SA share 0% to 100%",
        ),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]
