"""Shapes of the DFlash2 block-drafter workloads.

The drafter's dimensions follow the config fields the drafter reads
(dflash2.ts diff on the @mlx-bun/inference page, `Dflash2Config` and
`readConfig`) and the constructor parameters of the MAX
`DFlash2Qwen3_5` class (block_size, conv_kernel_size, conv_group_size,
selector_rank, selector_top_k).  Only two-tap convolutions exist there
(`readConfig` rejects any other conv_kernel_size), so `conv_taps` is fixed at 2.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class DrafterDims:
    hidden: int            # H
    layers: int
    heads: int             # NH
    kv_heads: int          # NKV
    head_dim: int          # D
    intermediate: int      # F (MLP width)
    n_taps: int            # target hidden-state taps concatenated into fc
    block_size: int        # G: the anchor row plus G-1 mask rows
    conv_group: int        # channels sharing one dynamic coefficient
    top_k: int             # K candidates per mask slot
    rank: int              # R, codebook rank of the selector
    vocab: int             # V
    rms_eps: float = 1e-6
    rope_theta: float = 1e7
    conv_taps: int = 2
    sliding_window: int = 0             # 0: every layer attends to all of its context
    sliding_layers: tuple | None = None # per-layer sliding flags; None: all layers slide

    @property
    def groups(self) -> int:
        return self.hidden // self.conv_group

    @property
    def qkv_width(self) -> int:
        return (self.heads + 2 * self.kv_heads) * self.head_dim


@dataclass(frozen=True)
class Workload:
    name: str
    dims: DrafterDims
    batch: int             # B anchors (requests)
    ctx_len: int           # L context rows per request
    seed: int              # base seed of the synthetic inputs
    kv_given: bool = False # context K/V supplied directly instead of from taps


TINY_DIMS = DrafterDims(hidden=256, layers=1, heads=4, kv_heads=2, head_dim=64,
                        intermediate=512, n_taps=2, block_size=8, conv_group=16,
                        top_k=4, rank=16, vocab=1024)

FULL_DIMS = DrafterDims(hidden=5120, layers=5, heads=32, kv_heads=8, head_dim=128,
                        intermediate=17408, n_taps=5, block_size=16, conv_group=16,
                        top_k=16, rank=64, vocab=248320)

# Tiny drafter: 1 layer, B=1, G=8, 32 context rows from 2 taps.
TINY = Workload("tiny", TINY_DIMS, batch=1, ctx_len=32, seed=1)
# Tiny drafter with a sliding layer followed by a full-attention layer: window of 20
# positions over 32 context rows, so block row t sees context rows 13 + t .. 31.
TINY_SW = Workload("tiny_sw", replace(TINY_DIMS, layers=2, sliding_window=20, sliding_layers=(True, False)),
                   batch=2, ctx_len=32, seed=6)
# Medium drafter: one layer whose gate/up projection (65536 x 1024 weights) is large enough
# for the weight-streaming GEMM; B=1, G=8, 32 context rows.
MEDIUM = Workload("medium", replace(TINY_DIMS, hidden=1024, heads=8, kv_heads=2, head_dim=128,
                                    intermediate=32768, vocab=2048, rank=32),
                  batch=1, ctx_len=32, seed=7)
# Full 5-layer drafter shaped like the 27B-target drafter: B=8, G=16, L=2048.
FULL = Workload("full", FULL_DIMS, batch=8, ctx_len=2048, seed=4)
# Long context, large batch: B=64, L=8192, context K/V given as N(0,1).
LONG = Workload("long", FULL_DIMS, batch=64, ctx_len=8192, seed=5, kv_given=True)

# Grouped dynamic conv microbench: [64*16, 5120] states, kernel_projection 5120 -> 1280.
CONV_BENCH = dict(name="conv", T=64 * 16, hidden=5120, block=16, group=16, seed=2)
# Candidate selector microbench: B=32, 15 slots, H=5120, K=16, V=248320, R=64.
SELECTOR_BENCH = dict(name="selector", B=32, S=15, hidden=5120, top_k=16,
                      vocab=248320, rank=64, seed=3)

WORKLOADS = {w.name: w for w in (TINY, FULL, LONG)}


def with_batch(w: Workload, batch: int, ctx_len: int | None = None) -> Workload:
    return replace(w, batch=batch, ctx_len=w.ctx_len if ctx_len is None else ctx_len)
