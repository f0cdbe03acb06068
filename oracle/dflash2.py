"""Plain CPU oracle of the DFlash2 block-drafter forward pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.  It shares
no code with the HIP library.

Every step is computed in float64 from the bf16 inputs (bf16 bit patterns are
widened exactly).  Where the pages fix a precision for a decision, the decision
is taken in that precision: candidate selection runs on float32 logits and the
walk on float32 scores (dflash2.ts diff on the @mlx-bun/inference page,
`#select`, casts the scores to fp32; MAX dflash2_qwen3_5 page, `compute_candidates`,
takes float32 logits).

Sources, cited by page title and section:
  [P1] codehub.bot function listing of the mirror-sd project: the neox RoPE and
       per-head RMSNorm docstrings.
  [P2] @mlx-bun/inference diff, dflash2.ts: header comment, `#rms`,
       `#coefficients`, `#conv`, `#rope`, `projectContext`, `#contextKV`,
       `#block`, `#select`.
  [P3] MAX Python API, max.pipelines.architectures.dflash2_qwen3_5:
       `DFlash2GroupedConv` (+ `prepare`, `finish`), `DFlash2CandidateSelector`
       (+ `score_edges`, `select_path`), `DFlash2Qwen3_5.compute_candidates`,
       `materialize`, `DFlash2TransformerBlock`.
  [P4] mlx-bun diff, qwen3_5.ts: the SwiGLU MLP of the target's layers.

Readings where the pages leave a step open (the numbered list of readings kept
with the design notes has the reasons):
  * RMSNorm: y = x / sqrt(mean(x^2) + eps) * gamma, gamma multiplies directly.
  * kernel_projection columns are ordered [side][tap][group], group fastest.
  * RoPE: neox split-half over all head_dim dims, inv_freq_i = theta^(-2i/D);
    context row j sits at position j, block row t at pos0[b] + t.
  * GQA: query head h reads KV head h // (NH / NKV).
  * Attention keys: every context row of the request, then the block's own G
    rows; no mask, no window; scale 1/sqrt(D).
  * Top-k order: value descending, then id ascending.  Walk ties: lowest slot.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


# ----------------------------------------------------------------------------
# number plumbing

def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        raise TypeError(f"expected bf16 bit patterns as uint16, got {b.dtype}")
    return (b.astype(np.uint32) << 16).view(np.float32).astype(F64)


def as_f64(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    return widen_bf16(a) if a.dtype == np.uint16 else a.astype(F64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16 value (ties to even), returned as float64.

    Used only by the optional `bf16_points` switch, which rounds activations at
    the points where [P2] `#block` casts back to bf16, for diagnosis.
    """
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return widen_bf16(u.astype(np.uint16))


def _maybe_round(x, on):
    return round_to_bf16(x) if on else x


# ----------------------------------------------------------------------------
# per-step functions

def rms_norm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis with a direct gain ([P2] `#rms`; [P1] per-head
    RMSNorm docstring for q/k with a [head_dim] weight)."""
    x = as_f64(x)
    g = as_f64(gamma)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * g


def rope_neox(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Neox (split-half) rotary embedding over all D dims ([P1] RoPE docstring:
    the rotated half is cat(-x[D/2:], x[:D/2]) and cos/sin are tiled over both
    halves; [P2] `#rope` rotates all head_dim dims).

    x: [rows, heads, D]; positions: [rows] absolute positions.
    """
    x = as_f64(x)
    D = x.shape[-1]
    half = D // 2
    i = np.arange(half, dtype=F64)
    inv_freq = theta ** (-(2.0 * i) / D)
    ang = np.asarray(positions, dtype=F64)[:, None] * inv_freq[None, :]      # [rows, D/2]
    cos = np.concatenate([np.cos(ang), np.cos(ang)], axis=-1)[:, None, :]    # [rows, 1, D]
    sin = np.concatenate([np.sin(ang), np.sin(ang)], axis=-1)[:, None, :]
    rotated = np.concatenate([-x[..., half:], x[..., :half]], axis=-1)
    return x * cos + rotated * sin


def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y = x . W^T for a weight stored [out, in] ([P2] `Bf16Projection`, which
    multiplies by the stored transpose)."""
    return as_f64(x) @ as_f64(w).T


def dequant_affine4(packed, scales, biases, group: int = 64, bf16_weights=False) -> np.ndarray:
    """Weights of a 4-bit affine projection ([P2] `quantizedWeight`: groups of 64 along the
    input dimension, affine mode, a scale and a bias per group):
    w[n, k] = scale[n, k // 64] * q[n, k] + bias[n, k // 64], q[n, k] in 0..15.

    packed: [N, K/8] uint32 (or int32 bit patterns); field k of row n sits at bits
    4 * (k % 8) of word k // 8, lowest bits first.  scales, biases: [N, K/64] bf16.
    `bf16_weights` rounds w to bf16, where a kernel feeding bf16 matrix units holds it.
    Returns float64 [N, K]."""
    p = np.asarray(packed).astype(np.int64) & 0xFFFFFFFF
    N, words = p.shape
    K = words * 8
    shifts = 4 * np.arange(8)
    q = ((p[:, :, None] >> shifts[None, None, :]) & 0xF).reshape(N, K).astype(F64)
    s = np.repeat(as_f64(scales), group, axis=1)
    b = np.repeat(as_f64(biases), group, axis=1)
    w = s * q + b
    return round_to_bf16(w) if bf16_weights else w


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def kernel_projection(n: np.ndarray, w_kp: np.ndarray) -> np.ndarray:
    """D = n . W_kp^T viewed as [T, side, tap, group] ([P2] header comment: one
    projection of the normed rows gives a delta per conv side, tap and channel group;
    [P3] `DFlash2GroupedConv`: its width is two sides times taps times groups, so both
    sides come from the one projection)."""
    T = n.shape[0]
    d = linear(n, w_kp)
    return d.reshape(T, 2, 2, -1)


def expand_groups(delta: np.ndarray, group: int) -> np.ndarray:
    """Per-group deltas [..., ng] -> per-channel [..., ng*group]: channel c takes
    group c // group ([P2] `#coefficients` broadcasts each group over its
    conv_group_size channels)."""
    return np.repeat(delta, group, axis=-1)


def conv_side(y: np.ndarray, coef: np.ndarray, block: int) -> np.ndarray:
    """One side of the two-tap conv along each block's rows ([P2] header conv
    equation and `#conv`; [P3] `DFlash2GroupedConv`: block-local, the t - tap
    term is zero at the first row of every block).

    y: [T, H] with T a multiple of `block`; coef: [T, 2 (tap), H], tap 0 weighs
    y[t] and tap 1 weighs y[t-1].
    """
    y = as_f64(y)
    T, H = y.shape
    if T % block:
        raise ValueError("rows must be whole blocks")
    yb = y.reshape(T // block, block, H)
    prev = np.zeros_like(yb)
    prev[:, 1:, :] = yb[:, :-1, :]
    cb = coef.reshape(T // block, block, 2, H)
    out = cb[:, :, 0, :] * yb + cb[:, :, 1, :] * prev
    return out.reshape(T, H)


def conv_prepare(x: np.ndarray, w_kp: np.ndarray, base: np.ndarray, block: int, group: int):
    """[P3] `DFlash2GroupedConv.prepare`: kernel_projection on the sublayer input,
    side 0 applied to that input; returns (convolved [T, H], side-1 deltas
    [T, taps, groups]).  The deltas exclude the base kernel (finish adds it)."""
    base = as_f64(base)                                   # [side, tap, H]
    d = kernel_projection(x, w_kp)                        # [T, side, tap, ng]
    coef0 = base[0][None, :, :] + expand_groups(d[:, 0], group)
    return conv_side(x, coef0, block), d[:, 1].copy()


def conv_finish(y: np.ndarray, deltas1: np.ndarray, base: np.ndarray, block: int, group: int):
    """[P3] `DFlash2GroupedConv.finish`: side 1 with the coefficients prepare()
    produced, on the sublayer's output."""
    base = as_f64(base)
    coef1 = base[1][None, :, :] + expand_groups(as_f64(deltas1), group)
    return conv_side(y, coef1, block)


def attention(q: np.ndarray, k_ctx: np.ndarray, v_ctx: np.ndarray, k_blk: np.ndarray,
              v_blk: np.ndarray, ctx_len: np.ndarray, pos0=None, window: int = 0) -> np.ndarray:
    """Bidirectional block attention over the request's context prefix plus the
    block's own rows ([P2] header comment: no causal mask inside the block; `#block`
    hands the block's k/v to the context's attend call with scale 1/sqrt(D)).

    window > 0 is a sliding-attention layer ([P3] `DFlash2Qwen3_5` `layer_types`;
    [P3] `construct_kv_params`: the drafter's mask reaches back at most the window):
    block row t of request b sits at position pos0[b] + t and sees context row j
    (position j) only when j >= pos0[b] + t - window + 1.  The block's own rows are
    always seen.

    q: [B, G, NH, D]; k_ctx, v_ctx: [B, Lcap, NKV, D]; k_blk, v_blk: [B, G, NKV, D];
    ctx_len: [B] context rows used per request.  Returns [B, G, NH, D].
    """
    q = as_f64(q)
    B, G, NH, D = q.shape
    NKV = k_blk.shape[2]
    rep = NH // NKV
    out = np.zeros_like(q)
    kc, vc, kb, vb = as_f64(k_ctx), as_f64(v_ctx), as_f64(k_blk), as_f64(v_blk)
    for b in range(B):
        L = int(ctx_len[b])
        keys = np.concatenate([kc[b, :L], kb[b]], axis=0)      # [L+G, NKV, D]
        vals = np.concatenate([vc[b, :L], vb[b]], axis=0)
        seen = np.ones((G, L + G), dtype=bool)
        if window > 0:
            first = int(pos0[b]) + np.arange(G) - window + 1    # first visible context row per block row
            seen[:, :L] = np.arange(L)[None, :] >= first[:, None]
        for h in range(NH):
            g = h // rep
            s = q[b, :, h, :] @ keys[:, g, :].T / np.sqrt(D)   # [G, L+G]
            s = np.where(seen, s, -np.inf)
            s = s - s.max(axis=-1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=-1, keepdims=True)
            out[b, :, h, :] = p @ vals[:, g, :]
    return out


def layer_window(dims, i: int) -> int:
    """Window of layer i: dims.sliding_window for a sliding layer, 0 for full attention
    ([P3] `layer_types`: None applies the window to every layer)."""
    w = getattr(dims, "sliding_window", 0) or 0
    kinds = getattr(dims, "sliding_layers", None)
    if w <= 0 or (kinds is not None and not kinds[i]):
        return 0
    return int(w)


def mlp(i: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray, bf16_points=False):
    """SwiGLU: down(silu(gate(i)) * up(i)) ([P2] `#block` MLP half; [P4] SwiGLU
    as silu(g) * u).  With `bf16_points`, g, u, silu(g) and the product are each
    rounded to bf16, as the bf16 ops of [P2] `#block` return them."""
    rnd = lambda a: _maybe_round(a, bf16_points)
    g = rnd(linear(i, w_gate))
    u = rnd(linear(i, w_up))
    prod = rnd(rnd(silu(g)) * u)
    return linear(prod, w_down)


# ----------------------------------------------------------------------------
# context and block

def project_context(taps: np.ndarray, w_fc: np.ndarray, hidden_norm: np.ndarray, eps: float,
                    bf16_points=False):
    """c = RMSNorm(fc(concat of the target taps)) with the hidden_norm gain ([P2] header
    comment and `projectContext`: the taps are concatenated, projected by fc and
    normalised; the bf16 fc output and norm output there are what `bf16_points` rounds).

    taps: [B, L, n_taps*H] with the taps concatenated on the feature axis.
    """
    rnd = lambda a: _maybe_round(a, bf16_points)
    return rnd(rms_norm(rnd(linear(taps, w_fc)), hidden_norm, eps))


def context_kv(c: np.ndarray, w_k: np.ndarray, w_v: np.ndarray, k_norm: np.ndarray,
               kv_heads: int, head_dim: int, eps: float, theta: float, positions=None,
               bf16_points=False):
    """One layer's context K/V: K = RoPE(k_norm(k_proj c)) at each row's absolute
    position, V = v_proj c; no input norm and no conv ([P2] `#contextKV`;
    [P3] `materialize`).  c: [B, L, H] -> K, V: [B, L, NKV, D].  `bf16_points`
    rounds the projection, norm and RoPE outputs, which [P2] holds in bf16."""
    rnd = lambda a: _maybe_round(a, bf16_points)
    B, L, _ = c.shape
    k = rnd(linear(c, w_k)).reshape(B, L, kv_heads, head_dim)
    v = rnd(linear(c, w_v)).reshape(B, L, kv_heads, head_dim)
    k = rnd(rms_norm(k, k_norm, eps))
    pos = np.arange(L) if positions is None else np.asarray(positions)
    kr = np.stack([rnd(rope_neox(k[b], pos, theta)) for b in range(B)], axis=0)
    return kr, v


def block_layer(x: np.ndarray, lw: dict, k_ctx, v_ctx, ctx_len, pos0, dims, bf16_points=False,
                window: int = 0):
    """One drafter layer on the block ([P3] `DFlash2TransformerBlock`: r = x;
    h = norm(r); h = conv.prepare(h); h = attn(h); h = conv.finish(h); r += h;
    the same for the MLP; [P2] `#block`, whose q/k norm precedes RoPE).

    x: [B, G, H] float64.  lw: this layer's tensors under their checkpoint names
    without the "layers.i." prefix.
    """
    B, G, H = x.shape
    NH, NKV, D = dims.heads, dims.kv_heads, dims.head_dim
    eps, theta, grp = dims.rms_eps, dims.rope_theta, dims.conv_group
    T = B * G
    rnd = lambda a: _maybe_round(a, bf16_points)
    positions = (np.asarray(pos0)[:, None] + np.arange(G)[None, :]).reshape(T)

    # attention half
    n = rnd(rms_norm(x.reshape(T, H), lw["input_layernorm.weight"], eps))
    a, d1 = conv_prepare(n, lw["attention_conv.kernel_projection.weight"],
                         lw["attention_conv.base_kernel"], G, grp)
    a = rnd(a)
    q = rnd(linear(a, lw["self_attn.q_proj.weight"])).reshape(T, NH, D)
    k = rnd(linear(a, lw["self_attn.k_proj.weight"])).reshape(T, NKV, D)
    v = rnd(linear(a, lw["self_attn.v_proj.weight"])).reshape(T, NKV, D)
    q = rnd(rope_neox(rnd(rms_norm(q, lw["self_attn.q_norm.weight"], eps)), positions, theta))
    k = rnd(rope_neox(rnd(rms_norm(k, lw["self_attn.k_norm.weight"], eps)), positions, theta))
    o = attention(q.reshape(B, G, NH, D), k_ctx, v_ctx, k.reshape(B, G, NKV, D),
                  v.reshape(B, G, NKV, D), ctx_len, pos0, window)
    o = rnd(o.reshape(T, NH * D))
    u = rnd(linear(o, lw["self_attn.o_proj.weight"]))
    xf = x.reshape(T, H) + conv_finish(u, d1, lw["attention_conv.base_kernel"], G, grp)
    xf = rnd(xf)

    # MLP half
    m = rnd(rms_norm(xf, lw["post_attention_layernorm.weight"], eps))
    i, d1m = conv_prepare(m, lw["mlp_conv.kernel_projection.weight"], lw["mlp_conv.base_kernel"], G, grp)
    i = rnd(i)
    f = rnd(mlp(i, lw["mlp.gate_proj.weight"], lw["mlp.up_proj.weight"], lw["mlp.down_proj.weight"],
                bf16_points))
    xf = rnd(xf + conv_finish(f, d1m, lw["mlp_conv.base_kernel"], G, grp))
    return xf.reshape(B, G, H)


def layer_weights(weights: dict, i: int) -> dict:
    p = f"layers.{i}."
    return {k[len(p):]: v for k, v in weights.items() if k.startswith(p)}


def materialize_context(taps, weights: dict, dims, positions=None, bf16_points=False):
    """Context K/V of every layer from the target taps ([P2] `projectContext` then
    `#contextKV`).  Returns lists K[layer], V[layer], each [B, L, NKV, D]."""
    c = project_context(taps, weights["fc.weight"], weights["hidden_norm.weight"], dims.rms_eps,
                        bf16_points)
    ks, vs = [], []
    for i in range(dims.layers):
        lw = layer_weights(weights, i)
        k, v = context_kv(c, lw["self_attn.k_proj.weight"], lw["self_attn.v_proj.weight"],
                          lw["self_attn.k_norm.weight"], dims.kv_heads, dims.head_dim,
                          dims.rms_eps, dims.rope_theta, positions, bf16_points)
        ks.append(k)
        vs.append(v)
    return ks, vs


def draft_hidden(embeds, weights: dict, k_ctx: list, v_ctx: list, ctx_len, pos0, dims,
                 bf16_points=False):
    """Rows 1..G-1 of the block after all layers and the final norm ([P2] `#block`:
    the anchor row is dropped, then `norm`).  Returns h [B, G-1, H]."""
    x = as_f64(embeds)
    for i in range(dims.layers):
        x = block_layer(x, layer_weights(weights, i), k_ctx[i], v_ctx[i], ctx_len, pos0, dims,
                        bf16_points, layer_window(dims, i))
    return _maybe_round(rms_norm(x[:, 1:, :], weights["norm.weight"], dims.rms_eps), bf16_points)


# ----------------------------------------------------------------------------
# candidate selector

def head_logits(h: np.ndarray, lm_head: np.ndarray) -> np.ndarray:
    """The target head over the drafter's normed rows ([P2] header: rows 1..G-1
    -> norm -> the target's lm_head); float64 here, float32 where it decides."""
    return linear(h, lm_head)


def compute_candidates(logits: np.ndarray, k: int):
    """Top-k ids per row and their logits ([P3] `compute_candidates`; [P2]
    `#select` partitions every position's scores once).  The list is ordered by
    value descending, then id ascending.  logits: [..., V] -> ids int32 [..., k],
    unary (same dtype as logits) [..., k]."""
    lg = np.asarray(logits)
    flat = lg.reshape(-1, lg.shape[-1])
    ids = np.empty((flat.shape[0], k), dtype=np.int32)
    for r in range(flat.shape[0]):
        row = flat[r]
        order = np.lexsort((np.arange(row.shape[0]), -row))   # primary: -value, then id
        ids[r] = order[:k]
    unary = np.take_along_axis(flat, ids.astype(np.int64), axis=1)
    return ids.reshape(*lg.shape[:-1], k), unary.reshape(*lg.shape[:-1], k)


def selector_project(h: np.ndarray, w_proj: np.ndarray) -> np.ndarray:
    """z = hidden_projection(h) ([P2] `#block`: z from the normed rows;
    [P3] `DFlash2CandidateSelector`: proj(h_l))."""
    return linear(h, w_proj)


def score_edges(cand: np.ndarray, unary: np.ndarray, z: np.ndarray, anchors: np.ndarray,
                pred: np.ndarray, succ: np.ndarray) -> np.ndarray:
    """S[b,l,p,c] = unary[b,l,c] + sum_r pred[pid(b,l,p), r] z[b,l,r] succ[cand[b,l,c], r]
    with pid(b,0,p) = anchor[b] and pid(b,l,p) = cand[b,l-1,p] for l >= 1
    ([P3] `DFlash2CandidateSelector` and `score_edges`).  Returns [B, S, K, K]."""
    cand = np.asarray(cand)
    B, S, K = cand.shape
    pb, sb = as_f64(pred), as_f64(succ)
    zz, un = as_f64(z), as_f64(unary)
    pid = np.empty((B, S, K), dtype=np.int64)
    pid[:, 0, :] = np.asarray(anchors)[:, None]
    pid[:, 1:, :] = cand[:, :-1, :]
    w = pb[pid] * zz[:, :, None, :]                  # [B, S, K(p), R]
    edge = np.einsum("blpr,blcr->blpc", w, sb[cand])
    return un[:, :, None, :] + edge


def select_path(scores: np.ndarray, cand: np.ndarray, seed_index: int = 0) -> np.ndarray:
    """Greedy left-to-right walk ([P3] `select_path`: one pass, no beam, slot 0
    seeded at any predecessor index; [P2] `#select`: argmax per position, the
    first maximum wins).  scores: [B, S, K, K] (decided in float32);
    returns tokens int32 [B, S]."""
    sc = np.asarray(scores, dtype=np.float32)
    cand = np.asarray(cand)
    B, S, K, _ = sc.shape
    out = np.empty((B, S), dtype=np.int32)
    for b in range(B):
        j = seed_index
        for l in range(S):
            row = sc[b, l, j]
            j = int(np.argmax(row))                  # first occurrence of the max
            out[b, l] = cand[b, l, j]
    return out


def draft_block(embeds, weights: dict, lm_head, anchors, k_ctx: list, v_ctx: list, ctx_len,
                pos0, dims, bf16_points=False, return_all=False, vocab_ids=None):
    """The whole block: layers, head, candidates, score_edges and the walk
    ([P2] `#block` and `#select`; [P3] `forward_block`, `compute_candidates`,
    `score_edges`, `select_path`).  Returns tokens [B, G-1] int32.

    vocab_ids: a draft vocabulary ([P2] `#block` and `#select`: a target that lists one is
    projected onto those rows of its head only, and the chosen columns map to the listed
    token ids before the path walk); None: the columns are the token ids."""
    h = draft_hidden(embeds, weights, k_ctx, v_ctx, ctx_len, pos0, dims, bf16_points)
    if vocab_ids is not None:
        vocab_ids = np.asarray(vocab_ids, dtype=np.int64)
        lm_head = np.asarray(lm_head)[vocab_ids]
    logits = head_logits(h, lm_head).astype(np.float32)
    cand, unary = compute_candidates(logits, dims.top_k)
    if vocab_ids is not None:
        cand = vocab_ids[cand].astype(np.int32)
    z = selector_project(h, weights["candidate_selector.hidden_projection.weight"])
    scores = score_edges(cand, unary, z, anchors, weights["candidate_selector.predecessor_codebook"],
                         weights["candidate_selector.successor_codebook"]).astype(np.float32)
    tokens = select_path(scores, cand)
    if return_all:
        return dict(h=h, logits=logits, cand=cand, unary=unary, z=z, scores=scores, tokens=tokens)
    return tokens
