"""Pins of how the oracle composes a drafter layer and the context projection.

The per-step functions are pinned elsewhere; these tests pin the order in which a layer
strings them together, with weights chosen so that the expected output has a closed form:

* MAX dflash2_qwen3_5 page, `DFlash2TransformerBlock`: each sublayer normalises the
  residual, runs the conv's prepare on the normed rows, the sublayer, the conv's finish,
  and adds the result to the residual; the attention half uses the input norm and the
  attention conv, the MLP half the post-attention norm and the MLP conv.
* Same page, `DFlash2GroupedConv`: the kernel projection reads the sublayer's input (the
  normed rows) once and yields both sides' deltas; prepare applies side 0, finish side 1
  with the deltas of the same rows.
* @mlx-bun/inference dflash2.ts diff, `#block`: q and k are normalised per head before
  RoPE; `projectContext`: the context rows are the fc output normalised with the
  hidden_norm gain.

A throwaway mutation of the oracle for each of these readings (finish taking side 0's
deltas, deltas computed from x instead of the normed rows, RoPE before the q/k norm, the
MLP half using the attention conv's weights, the context normalised with `norm` instead of
`hidden_norm`) fails at least one test here.
"""
import dataclasses

import numpy as np
import pytest

from dflash2_block_drafter_amd import configs
from oracle import dflash2 as O

# A drafter small enough to write weights by hand: H = 32 channels in two conv groups of
# 16, two query heads sharing one KV head of 16 dims, blocks of 4 rows.
DIMS = configs.DrafterDims(hidden=32, layers=1, heads=2, kv_heads=1, head_dim=16, intermediate=24,
                           n_taps=2, block_size=4, conv_group=16, top_k=2, rank=4, vocab=16)
H, NH, NKV, D, F, G, NG = 32, 2, 1, 16, 24, 4, 2
EPS = DIMS.rms_eps


def _rms(x, g):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + EPS) * g


def _col(side, tap, g):
    """kernel_projection output column of (side, tap, group): [side][tap][group], group
    fastest (dflash2.ts diff, `#coefficients`)."""
    return (side * 2 + tap) * NG + g


def _layer_weights(rng):
    """Random nonzero weights for every tensor of one layer; tests overwrite some."""
    lw = {
        "input_layernorm.weight": 1.0 + 0.4 * rng.standard_normal(H),
        "post_attention_layernorm.weight": 1.0 + 0.4 * rng.standard_normal(H),
        "self_attn.q_proj.weight": 0.3 * rng.standard_normal((NH * D, H)),
        "self_attn.k_proj.weight": 0.3 * rng.standard_normal((NKV * D, H)),
        "self_attn.v_proj.weight": 0.3 * rng.standard_normal((NKV * D, H)),
        "self_attn.o_proj.weight": 0.3 * rng.standard_normal((H, NH * D)),
        "self_attn.q_norm.weight": 1.0 + 0.5 * rng.standard_normal(D),
        "self_attn.k_norm.weight": 1.0 + 0.5 * rng.standard_normal(D),
        "mlp.gate_proj.weight": 0.3 * rng.standard_normal((F, H)),
        "mlp.up_proj.weight": 0.3 * rng.standard_normal((F, H)),
        "mlp.down_proj.weight": 0.3 * rng.standard_normal((H, F)),
        "attention_conv.base_kernel": 0.5 + 0.1 * rng.standard_normal((2, 2, H)),
        "attention_conv.kernel_projection.weight": 0.1 * rng.standard_normal((4 * NG, H)),
        "mlp_conv.base_kernel": 0.5 + 0.1 * rng.standard_normal((2, 2, H)),
        "mlp_conv.kernel_projection.weight": 0.1 * rng.standard_normal((4 * NG, H)),
    }
    return lw


def _context(rng, B, L):
    return (rng.standard_normal((B, L, NKV, D)), rng.standard_normal((B, L, NKV, D)))


def test_attention_half_conv_reads_normed_input_and_finish_takes_side_one():
    """q = k = 0 makes attention uniform over the request's context rows and the block rows,
    so every row of request b gets the same u_b = W_o (mean of the attended V).  The
    attention conv's kernel projection is one-hot: side 1 tap 0 of every group reads
    alpha * n[t, c0], side 1 tap 1 reads alpha1 * n[t, c1], side 0 reads nothing, and base
    side 0 is (1, 0), so prepare passes n through.  With the MLP's down projection zero the
    layer output is
        x[t] + (beta + alpha n[t, c0]) u_b + (beta1 + alpha1 n[t, c1]) u_b [t % G != 0]
    with n = RMSNorm(x; input_layernorm)."""
    rng = np.random.default_rng(101)
    B, L = 2, 5
    lw = _layer_weights(rng)
    lw["self_attn.q_proj.weight"][:] = 0.0
    lw["self_attn.k_proj.weight"][:] = 0.0
    lw["mlp.down_proj.weight"][:] = 0.0
    c0, c1, alpha, alpha1 = 3, 20, 0.7, -0.45
    kp = np.zeros((4 * NG, H))
    for g in range(NG):
        kp[_col(1, 0, g), c0] = alpha
        kp[_col(1, 1, g), c1] = alpha1
    lw["attention_conv.kernel_projection.weight"] = kp
    base = np.empty((2, 2, H))
    base[0, 0], base[0, 1] = 1.0, 0.0
    beta, beta1 = 0.5 + 0.2 * rng.standard_normal(H), -0.3 + 0.2 * rng.standard_normal(H)
    base[1, 0], base[1, 1] = beta, beta1
    lw["attention_conv.base_kernel"] = base
    x = rng.standard_normal((B, G, H)) * 1.7
    kc, vc = _context(rng, B, L)
    ctx_len = np.array([L, 2])
    pos0 = ctx_len.copy()

    got = O.block_layer(x, lw, kc, vc, ctx_len, pos0, DIMS)

    n = _rms(x, lw["input_layernorm.weight"])                    # [B, G, H]
    want = np.empty_like(x)
    for b in range(B):
        v_blk = n[b] @ lw["self_attn.v_proj.weight"].T               # a = n: prepare is the identity
        keys_v = np.concatenate([vc[b, :ctx_len[b], 0], v_blk], axis=0)
        o = np.tile(keys_v.mean(axis=0), NH)                         # every head reads KV head 0
        u = lw["self_attn.o_proj.weight"] @ o
        for t in range(G):
            want[b, t] = x[b, t] + (beta + alpha * n[b, t, c0]) * u
            if t > 0:
                want[b, t] += (beta1 + alpha1 * n[b, t, c1]) * u
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_mlp_half_uses_its_own_norm_and_conv():
    """With o_proj zero the attention half adds nothing, so the MLP half sees x.  Its conv
    has one-hot deltas on both sides (side 0 tap 0 reads alpha2 * m[t, c2]; side 1 tap 0
    reads alpha3 * m[t, c3]) and its own base kernel; the attention conv carries very
    different weights that must not be used.  Expected, with m = RMSNorm(x;
    post_attention_layernorm):
        i[t] = (b00 + alpha2 m[t, c2]) m[t] + b01 m[t-1] [t % G != 0]
        f[t] = W_down (silu(W_gate i[t]) * W_up i[t])
        out[t] = x[t] + (b10 + alpha3 m[t, c3]) f[t] + b11 f[t-1] [t % G != 0]."""
    rng = np.random.default_rng(202)
    B, L = 2, 3
    lw = _layer_weights(rng)
    lw["self_attn.o_proj.weight"][:] = 0.0
    lw["attention_conv.base_kernel"] = np.stack([np.full((2, H), 5.0), np.full((2, H), -3.0)])
    lw["attention_conv.kernel_projection.weight"] = np.full((4 * NG, H), 0.9)
    c2, c3, alpha2, alpha3 = 30, 9, -0.6, 0.8
    kp = np.zeros((4 * NG, H))
    for g in range(NG):
        kp[_col(0, 0, g), c2] = alpha2
        kp[_col(1, 0, g), c3] = alpha3
    lw["mlp_conv.kernel_projection.weight"] = kp
    bm = 0.5 + 0.2 * rng.standard_normal((2, 2, H))
    lw["mlp_conv.base_kernel"] = bm
    x = rng.standard_normal((B, G, H)) * 0.8 + 0.3
    kc, vc = _context(rng, B, L)
    ctx = np.array([L, L])

    got = O.block_layer(x, lw, kc, vc, ctx, ctx, DIMS)

    m = _rms(x, lw["post_attention_layernorm.weight"])
    silu = lambda z: z / (1.0 + np.exp(-z))
    want = np.empty_like(x)
    for b in range(B):
        i = np.empty((G, H))
        for t in range(G):
            i[t] = (bm[0, 0] + alpha2 * m[b, t, c2]) * m[b, t]
            if t > 0:
                i[t] += bm[0, 1] * m[b, t - 1]
        f = (silu(i @ lw["mlp.gate_proj.weight"].T) * (i @ lw["mlp.up_proj.weight"].T)) @ lw["mlp.down_proj.weight"].T
        for t in range(G):
            want[b, t] = x[b, t] + (bm[1, 0] + alpha3 * m[b, t, c3]) * f[t]
            if t > 0:
                want[b, t] += bm[1, 1] * f[t - 1]
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_mlp_half_normalises_the_attention_half_output():
    """The post-attention norm reads the residual after the attention half, not the layer
    input: with the attention half of the first test active and a one-hot MLP conv that
    reads the normed residual, the MLP half's contribution follows m = RMSNorm(x1)."""
    rng = np.random.default_rng(303)
    B, L = 1, 4
    lw = _layer_weights(rng)
    lw["self_attn.q_proj.weight"][:] = 0.0
    lw["self_attn.k_proj.weight"][:] = 0.0
    base_a = np.zeros((2, 2, H))
    base_a[0, 0] = 1.0
    base_a[1, 0] = 1.0                        # finish adds u itself at every row
    lw["attention_conv.base_kernel"] = base_a
    lw["attention_conv.kernel_projection.weight"] = np.zeros((4 * NG, H))
    base_m = np.zeros((2, 2, H))
    base_m[0, 0] = 1.0                        # prepare passes m through
    lw["mlp_conv.base_kernel"] = base_m
    c4, alpha4 = 17, 1.3
    kp = np.zeros((4 * NG, H))
    for g in range(NG):
        kp[_col(1, 0, g), c4] = alpha4       # finish scales f[t] by alpha4 * m[t, c4]
    lw["mlp_conv.kernel_projection.weight"] = kp
    x = rng.standard_normal((B, G, H))
    kc, vc = _context(rng, B, L)
    ctx = np.array([L])

    got = O.block_layer(x, lw, kc, vc, ctx, ctx, DIMS)

    n = _rms(x[0], lw["input_layernorm.weight"])
    keys_v = np.concatenate([vc[0, :, 0], n @ lw["self_attn.v_proj.weight"].T], axis=0)
    u = lw["self_attn.o_proj.weight"] @ np.tile(keys_v.mean(axis=0), NH)
    x1 = x[0] + u[None, :]
    m = _rms(x1, lw["post_attention_layernorm.weight"])
    silu = lambda z: z / (1.0 + np.exp(-z))
    f = (silu(m @ lw["mlp.gate_proj.weight"].T) * (m @ lw["mlp.up_proj.weight"].T)) @ lw["mlp.down_proj.weight"].T
    want = x1 + alpha4 * m[:, c4:c4 + 1] * f
    assert np.allclose(got[0], want, rtol=1e-12, atol=1e-12)


def _shifted_layer(rng_seed, shift, lw=None):
    """A random layer run on a context materialised at positions shift + j and a block at
    position shift + L: with q/k normalised before RoPE, attention depends only on position
    differences, so the output does not depend on the shift."""
    rng = np.random.default_rng(rng_seed)
    B, L = 2, 6
    d = dataclasses.replace(DIMS, rope_theta=100.0)   # small theta: every pair rotates visibly
    if lw is None:
        lw = _layer_weights(rng)
    else:
        _layer_weights(rng)
    c = rng.standard_normal((B, L, H))
    x = rng.standard_normal((B, G, H))
    k, v = O.context_kv(c, lw["self_attn.k_proj.weight"], lw["self_attn.v_proj.weight"],
                        lw["self_attn.k_norm.weight"], NKV, D, EPS, d.rope_theta, positions=np.arange(L) + shift)
    ctx = np.array([L, L])
    return O.block_layer(x, lw, k, v, ctx, ctx + shift, d), lw


def test_layer_depends_on_relative_positions_only():
    """RoPE after the per-head norm makes q.k depend only on the two positions' difference,
    for any per-head gain.  Normalising after RoPE with a gain whose rotary pairs differ
    (gamma_i != gamma_{i + D/2}) would break that, so shifting every position changes
    nothing only under the norm-then-RoPE order."""
    base, lw = _shifted_layer(404, 0)
    g = lw["self_attn.q_norm.weight"]
    assert np.max(np.abs(g[:D // 2] - g[D // 2:])) > 0.1       # the gain is not pair-symmetric
    for shift in (1, 7, 1000):
        got, _ = _shifted_layer(404, shift, lw)
        assert np.allclose(got, base, rtol=1e-9, atol=1e-9), shift


def test_block_position_matters():
    """The converse: moving only the block (pos0) against a fixed context changes the output,
    so the shift test above is not vacuous."""
    rng = np.random.default_rng(505)
    B, L = 1, 6
    d = dataclasses.replace(DIMS, rope_theta=100.0)
    lw = _layer_weights(rng)
    c = rng.standard_normal((B, L, H))
    x = rng.standard_normal((B, G, H))
    k, v = O.context_kv(c, lw["self_attn.k_proj.weight"], lw["self_attn.v_proj.weight"],
                        lw["self_attn.k_norm.weight"], NKV, D, EPS, d.rope_theta)
    ctx = np.array([L])
    a = O.block_layer(x, lw, k, v, ctx, ctx, d)
    b = O.block_layer(x, lw, k, v, ctx, ctx + 3, d)
    assert np.max(np.abs(a - b)) > 1e-3


def test_project_context_hand_value_uses_hidden_norm():
    """fc = [I | 2I] makes the fc output tap1 + 2 tap2; the context rows are that, RMS
    normalised with the hidden_norm gain.  Through materialize_context with v_proj = [I | 0]
    the V cache of every layer is the first NKV*D channels of those rows, so a context
    normalised with `norm` (a very different gain here) would show."""
    rng = np.random.default_rng(606)
    B, L = 2, 3
    taps = rng.standard_normal((B, L, 2 * H))
    fc = np.concatenate([np.eye(H), 2.0 * np.eye(H)], axis=1)
    g_hidden = 1.0 + 0.5 * rng.standard_normal(H)
    raw = taps[..., :H] + 2.0 * taps[..., H:]
    want = raw / np.sqrt(np.mean(raw * raw, axis=-1, keepdims=True) + EPS) * g_hidden
    assert np.allclose(O.project_context(taps, fc, g_hidden, EPS), want, rtol=1e-13, atol=1e-13)

    lw = _layer_weights(rng)
    lw["self_attn.v_proj.weight"] = np.concatenate([np.eye(NKV * D), np.zeros((NKV * D, H - NKV * D))], axis=1)
    weights = {f"layers.0.{k}": v for k, v in lw.items()}
    weights["fc.weight"] = fc
    weights["hidden_norm.weight"] = g_hidden
    weights["norm.weight"] = -3.0 * np.ones(H)
    ks, vs = O.materialize_context(taps, weights, DIMS)
    assert np.allclose(vs[0].reshape(B, L, NKV * D), want[..., :NKV * D], rtol=1e-13, atol=1e-13)


def test_draft_hidden_drops_anchor_and_uses_final_norm():
    """With o_proj and down_proj zero both sublayers add nothing, so the hidden rows the head
    reads are rows 1..G-1 of the embedded block, RMS normalised with the `norm` gain
    (dflash2.ts diff, `#block`: the anchor row is dropped before the final norm)."""
    rng = np.random.default_rng(707)
    B, L = 2, 3
    lw = _layer_weights(rng)
    lw["self_attn.o_proj.weight"][:] = 0.0
    lw["mlp.down_proj.weight"][:] = 0.0
    weights = {f"layers.0.{k}": v for k, v in lw.items()}
    g_final = 1.0 + 0.5 * rng.standard_normal(H)
    weights["norm.weight"] = g_final
    x = rng.standard_normal((B, G, H))
    kc, vc = _context(rng, B, L)
    ctx = np.array([L, L])
    h = O.draft_hidden(x, weights, [kc], [vc], ctx, ctx, DIMS)
    assert h.shape == (B, G - 1, H)
    assert np.allclose(h, _rms(x[:, 1:], g_final), rtol=1e-13, atol=1e-13)
