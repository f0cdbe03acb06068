"""Seeded synthetic inputs for the drafter workloads.

This module only draws numbers: it holds none of the drafter's arithmetic and is
the one piece that both the HIP path's callers and the CPU oracle's callers use,
so that the two sides see the same bits.

Recipe (every tensor): a `torch.Generator` on the device the tensor will live on,
seeded with `seed_for(workload_seed, name)`; fp32 samples from `torch.randn`
(or `torch.rand` for ids), affine-mapped to the stated mean and standard
deviation, then rounded to bf16 by torch's round-to-nearest-even conversion.
The same seed on another device draws different numbers; a comparison always
copies one draw to the other side rather than drawing twice.

Distributions (second parameter = standard deviation):
  projection matrices, lm_head            N(0, 0.02)
  RMSNorm gains                           1 + N(0, 0.02)
  conv base kernels                       N(0.5, 0.1)
  selector codebooks                      N(0, 0.05)
  target taps, embedded rows, given K/V   N(0, 1)
  selector-bench logits (fp32)            N(0, 3)
  anchor ids                              uniform over [0, V)
"""
from __future__ import annotations

import zlib

import numpy as np
import torch

from .configs import DrafterDims, Workload


def seed_for(base: int, name: str) -> int:
    return (int(base) * 1_000_003 + zlib.crc32(name.encode())) & 0x7FFF_FFFF_FFFF


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, mean: float, std: float, *, seed: int, device="cpu",
           dtype=torch.bfloat16) -> torch.Tensor:
    g = _gen(device, seed)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x.to(dtype)


def uniform_ids(n: int, high: int, *, seed: int, device="cpu") -> torch.Tensor:
    g = _gen(device, seed)
    return torch.randint(0, high, (n,), generator=g, device=device, dtype=torch.int32)


def layer_names(i: int) -> list[str]:
    p = f"layers.{i}"
    return [f"{p}.input_layernorm.weight", f"{p}.post_attention_layernorm.weight",
            f"{p}.self_attn.q_proj.weight", f"{p}.self_attn.k_proj.weight",
            f"{p}.self_attn.v_proj.weight", f"{p}.self_attn.o_proj.weight",
            f"{p}.self_attn.q_norm.weight", f"{p}.self_attn.k_norm.weight",
            f"{p}.mlp.gate_proj.weight", f"{p}.mlp.up_proj.weight", f"{p}.mlp.down_proj.weight",
            f"{p}.attention_conv.base_kernel", f"{p}.attention_conv.kernel_projection.weight",
            f"{p}.mlp_conv.base_kernel", f"{p}.mlp_conv.kernel_projection.weight"]


def weight_specs(d: DrafterDims) -> dict[str, tuple[tuple[int, ...], float, float]]:
    """Checkpoint tensor name -> (shape, mean, std), with the drafter's checkpoint names."""
    H, NH, NKV, D, F, ng = d.hidden, d.heads, d.kv_heads, d.head_dim, d.intermediate, d.groups
    gain = (1.0, 0.02)
    proj = (0.0, 0.02)
    specs: dict[str, tuple[tuple[int, ...], float, float]] = {
        "fc.weight": ((H, d.n_taps * H), *proj),
        "hidden_norm.weight": ((H,), *gain),
        "norm.weight": ((H,), *gain),
        "candidate_selector.hidden_projection.weight": ((d.rank, H), *proj),
        "candidate_selector.predecessor_codebook": ((d.vocab, d.rank), 0.0, 0.05),
        "candidate_selector.successor_codebook": ((d.vocab, d.rank), 0.0, 0.05),
    }
    for i in range(d.layers):
        p = f"layers.{i}"
        specs.update({
            f"{p}.input_layernorm.weight": ((H,), *gain),
            f"{p}.post_attention_layernorm.weight": ((H,), *gain),
            f"{p}.self_attn.q_proj.weight": ((NH * D, H), *proj),
            f"{p}.self_attn.k_proj.weight": ((NKV * D, H), *proj),
            f"{p}.self_attn.v_proj.weight": ((NKV * D, H), *proj),
            f"{p}.self_attn.o_proj.weight": ((H, NH * D), *proj),
            f"{p}.self_attn.q_norm.weight": ((D,), *gain),
            f"{p}.self_attn.k_norm.weight": ((D,), *gain),
            f"{p}.mlp.gate_proj.weight": ((F, H), *proj),
            f"{p}.mlp.up_proj.weight": ((F, H), *proj),
            f"{p}.mlp.down_proj.weight": ((H, F), *proj),
            f"{p}.attention_conv.base_kernel": ((2, 2, H), 0.5, 0.1),
            f"{p}.attention_conv.kernel_projection.weight": ((4 * ng, H), *proj),
            f"{p}.mlp_conv.base_kernel": ((2, 2, H), 0.5, 0.1),
            f"{p}.mlp_conv.kernel_projection.weight": ((4 * ng, H), *proj),
        })
    return specs


def drafter_weights(w: Workload, device="cpu") -> dict[str, torch.Tensor]:
    out = {}
    for name, (shape, mean, std) in weight_specs(w.dims).items():
        out[name] = normal(shape, mean, std, seed=seed_for(w.seed, name), device=device)
    return out


def target_inputs(w: Workload, device="cpu", *, with_taps: bool = True) -> dict[str, torch.Tensor]:
    """The target-owned tensors the drafter borrows, plus the per-request inputs.

    embeds[b, 0] is the embedded anchor and embeds[b, t>=1] the embedded mask
    token (one shared row), as the target's embedding would give them.
    """
    d, B, L, G, H = w.dims, w.batch, w.ctx_len, w.dims.block_size, w.dims.hidden
    s = w.seed
    anchor_rows = normal((B, 1, H), 0.0, 1.0, seed=seed_for(s, "embed.anchor"), device=device)
    mask_row = normal((1, 1, H), 0.0, 1.0, seed=seed_for(s, "embed.mask"), device=device)
    embeds = torch.cat([anchor_rows, mask_row.expand(B, G - 1, H)], dim=1).contiguous()
    out = {
        "lm_head": normal((d.vocab, H), 0.0, 0.02, seed=seed_for(s, "lm_head"), device=device),
        "embeds": embeds,
        "anchors": uniform_ids(B, d.vocab, seed=seed_for(s, "anchors"), device=device),
        "ctx_len": torch.full((B,), L, dtype=torch.int32, device=device),
        "pos0": torch.full((B,), L, dtype=torch.int32, device=device),
    }
    if with_taps and not w.kv_given:
        out["taps"] = normal((B, L, d.n_taps * H), 0.0, 1.0, seed=seed_for(s, "taps"), device=device)
    return out


def given_kv(w: Workload, layer: int, device="cpu") -> tuple[torch.Tensor, torch.Tensor]:
    """Context K/V supplied directly, [B, L, NKV, D] bf16 N(0, 1) each."""
    d = w.dims
    shape = (w.batch, w.ctx_len, d.kv_heads, d.head_dim)
    k = normal(shape, 0.0, 1.0, seed=seed_for(w.seed, f"ctx.k.{layer}"), device=device)
    v = normal(shape, 0.0, 1.0, seed=seed_for(w.seed, f"ctx.v.{layer}"), device=device)
    return k, v


def selector_inputs(B: int, S: int, H: int, K: int, V: int, R: int, seed: int,
                    device="cpu", logit_std: float = 3.0, book_std: float = 0.05):
    """Inputs of the candidate-selector microbench."""
    return {
        "logits": normal((B, S, V), 0.0, logit_std, seed=seed_for(seed, "logits"), device=device,
                         dtype=torch.float32),
        "hidden": normal((B, S, H), 0.0, 1.0, seed=seed_for(seed, "hidden"), device=device),
        "proj": normal((R, H), 0.0, 0.02, seed=seed_for(seed, "proj"), device=device),
        "pred": normal((V, R), 0.0, book_std, seed=seed_for(seed, "pred"), device=device),
        "succ": normal((V, R), 0.0, book_std, seed=seed_for(seed, "succ"), device=device),
        "anchors": uniform_ids(B, V, seed=seed_for(seed, "anchors"), device=device),
    }


def conv_inputs(T: int, H: int, grp: int, seed: int, device="cpu"):
    """Inputs of the grouped-conv microbench."""
    ng = H // grp
    return {
        "x": normal((T, H), 0.0, 1.0, seed=seed_for(seed, "x"), device=device),
        "kproj": normal((4 * ng, H), 0.0, 0.02, seed=seed_for(seed, "kproj"), device=device),
        "base": normal((2, 2, H), 0.5, 0.1, seed=seed_for(seed, "base"), device=device),
    }


def affine4_weight(N: int, K: int, *, seed: int, device="cpu"):
    """A 4-bit affine projection of N rows over K inputs (groups of 64): packed int32 words
    [N, K/8] of uniform 4-bit fields, scales [N, K/64] ~ |N(0.003, 0.001)| and biases
    = -7.5 * scale + N(0, 0.002), both bf16, so the weights span about +-0.02 around 0."""
    g = _gen(device, seed)
    q = torch.randint(0, 16, (N, K // 8, 8), generator=g, dtype=torch.int64, device=device)
    words = (q << (4 * torch.arange(8, dtype=torch.int64, device=device))).sum(-1)
    del q
    words = torch.where(words >= 2 ** 31, words - 2 ** 32, words).to(torch.int32)
    scales = (torch.randn((N, K // 64), generator=g, device=device) * 0.001 + 0.003).abs().to(torch.bfloat16)
    biases = (-7.5 * scales.float() + torch.randn((N, K // 64), generator=g, device=device) * 0.002).to(torch.bfloat16)
    return words, scales, biases


def q4_projection_shapes(d: DrafterDims, i: int) -> dict[str, tuple[int, int]]:
    """The seven projections of layer i that a 4-bit drafter quantizes: checkpoint name
    without ".weight" -> (N, K)."""
    H, NH, NKV, D, F = d.hidden, d.heads, d.kv_heads, d.head_dim, d.intermediate
    p = f"layers.{i}"
    return {f"{p}.self_attn.q_proj": (NH * D, H), f"{p}.self_attn.k_proj": (NKV * D, H),
            f"{p}.self_attn.v_proj": (NKV * D, H), f"{p}.self_attn.o_proj": (H, NH * D),
            f"{p}.mlp.gate_proj": (F, H), f"{p}.mlp.up_proj": (F, H), f"{p}.mlp.down_proj": (H, F)}


def drafter_q4_weights(w: Workload, device="cpu") -> dict[str, tuple[torch.Tensor, torch.Tensor, torch.Tensor]]:
    """4-bit affine layer projections (affine4_weight each, seeded by name)."""
    out = {}
    for i in range(w.dims.layers):
        for name, (N, K) in q4_projection_shapes(w.dims, i).items():
            out[name] = affine4_weight(N, K, seed=seed_for(w.seed, name + ".q4"), device=device)
    return out


def bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a bf16 tensor as its raw uint16 bit patterns."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    """Host copy of any tensor; bf16 tensors come back as uint16 bit patterns."""
    if t.dtype == torch.bfloat16:
        return bits(t)
    return t.detach().contiguous().cpu().numpy()
