"""Element-by-element parity of every kernel the draft path launches, in the launch
configuration bench.py times (bound head, materialised or given context), at the tiny and
the full workload sizes.

dfl_draft_block_traced runs the same launch sequence as dfl_draft_block and copies each
stage's output; each stage is compared with the oracle computed from the GPU's own input to
that stage, so every kernel is held to the bar of one bf16-in / fp32-accumulate step
(|g - o| <= 2e-3 + 2e-2 |o|), fp32 plane copies and tile maxima bit for bit, score_edges at
1e-5 and the candidates and the walk bit for bit.  Cheap stages are checked on every row;
the projections and attention on the rows of two sampled requests (the first and the last).
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

from dflash2_block_drafter_amd import binding as B_
from dflash2_block_drafter_amd import configs, synth
from dflash2_block_drafter_amd.drafter import Drafter
from oracle import dflash2 as O
from tests.helpers import assert_bf16_close, assert_f32_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(f"[stages] {msg}", flush=True)


def f64(t):
    """Host float64 copy of a device tensor (bf16 widened exactly)."""
    return O.as_f64(synth.host(t))


def _stage_buffers(d, Bq, G, cols):
    T, N, H = Bq * G, Bq * (G - 1), d.hidden
    ng, qkvw, F, K, R = d.groups, d.qkv_width, d.intermediate, d.top_k, d.rank
    ntiles = (cols + 255) // 256
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    shapes = {"x_in": ((T, H), bf), "n": ((T, H), bf), "coef": ((T, 4 * ng), f32), "a": ((T, H), bf),
              "coef1": ((T, 2 * ng), f32), "qkv": ((T, qkvw), bf), "attn": ((T, d.heads * d.head_dim), bf),
              "u": ((T, H), bf), "x_mid": ((T, H), bf), "m": ((T, H), bf), "coef_mlp": ((T, 4 * ng), f32),
              "i": ((T, H), bf), "coef1_mlp": ((T, 2 * ng), f32), "p": ((T, F), bf), "f": ((T, H), bf),
              "x_out": ((T, H), bf), "n_next": ((T, H), bf), "h": ((N, H), bf), "tile_max": ((N, ntiles), f32),
              "cand": ((N, K), i32), "unary": ((N, K), f32), "z": ((N, R), f32), "scores": ((N, K, K), f32)}
    out = {}
    for k, (shape, dt) in shapes.items():
        # unwritten stages stay NaN (or -1) and fail the comparison
        out[k] = torch.full(shape, -1 if dt == i32 else float("nan"), dtype=dt, device=DEV)
    return out


class Run:
    """One workload on the GPU, set up as bench.py sets it up."""

    def __init__(self, w):
        self.w = w
        d = self.d = w.dims
        self.Bq, self.G, self.L = w.batch, d.block_size, w.ctx_len
        say(f"{w.name}: B={self.Bq} G={self.G} L={self.L} H={d.hidden} V={d.vocab}")
        self.weights = synth.drafter_weights(w, device=DEV)
        self.tgt = synth.target_inputs(w, device=DEV, with_taps=not w.kv_given)
        self.dr = Drafter(d, self.weights)
        if w.kv_given:
            self.K, self.V = [], []
            for i in range(d.layers):
                k, v = synth.given_kv(w, i, device=DEV)
                self.K.append(k)
                self.V.append(v)
        else:
            self.K, self.V = self.dr.alloc_kv(self.Bq, self.L)
            self.dr.materialize(self.tgt["taps"], self.K, self.V)
        self.dr.bind_target(self.tgt["lm_head"])
        self.ws = self.dr.workspace(self.Bq, self.G, self.L)
        self.wh = {}

    def host_weight(self, name):
        if name not in self.wh:
            self.wh[name] = synth.host(self.weights[name])
        return self.wh[name]

    def traced(self, layer):
        d = self.d
        st = _stage_buffers(d, self.Bq, self.G, d.vocab)
        tokens = torch.full((self.Bq, self.G - 1), -1, dtype=torch.int32, device=DEV)
        logits = torch.full((self.Bq, self.G - 1, d.vocab), float("nan"), dtype=torch.float32, device=DEV)
        B_.dfl_draft_block_traced(self.dr.handle, self.tgt["embeds"], self.tgt["anchors"], self.Bq, self.G, self.K,
                                  self.V, self.L, self.L, self.tgt["ctx_len"], self.tgt["pos0"], None, tokens, logits,
                                  self.ws, layer, st)
        torch.cuda.synchronize()
        # the traced call drafts exactly what the plain one drafts
        t2 = self.dr.draft(self.tgt["embeds"], self.tgt["anchors"], self.K, self.V, self.L, self.tgt["ctx_len"],
                           self.tgt["pos0"], None, ws=self.ws)
        torch.cuda.synchronize()
        assert torch.equal(tokens, t2)
        return st, tokens, logits

    def close(self):
        self.dr.close()


_RUNS = {}


def _run(name):
    if name not in _RUNS:
        for other in list(_RUNS):          # one large workload resident at a time
            _RUNS.pop(other).close()
        torch.cuda.empty_cache()
        w = {"tiny3": configs.with_batch(configs.TINY, 3), "tiny_sw": configs.TINY_SW,
             "full": configs.FULL, "long": configs.LONG}[name]
        _RUNS[name] = Run(w)
    return _RUNS[name]


@pytest.fixture(scope="module", autouse=True)
def _cleanup():
    yield
    for r in _RUNS.values():
        r.close()
    _RUNS.clear()
    torch.cuda.empty_cache()


def _conv(y, coef_side, base_side, d, G):
    """One conv side: coef_side [T, 2*ng] fp32 deltas (tap 0 groups, then tap 1)."""
    T = y.shape[0]
    delta = O.expand_groups(coef_side.reshape(T, 2, d.groups), d.conv_group)
    return O.conv_side(y, base_side[None, :, :] + delta, G)


def _rows_of(reqs, G):
    return np.concatenate([np.arange(b * G, (b + 1) * G) for b in reqs])


def check_layer(run, li, st):
    d, G, Bq = run.d, run.G, run.Bq
    T, H, ng = Bq * G, d.hidden, d.groups
    NH, NKV, D = d.heads, d.kv_heads, d.head_dim
    p = f"layers.{li}."
    W = lambda n: run.host_weight(p + n)
    reqs = sorted({0, Bq - 1})
    rows = _rows_of(reqs, G)
    pos0 = synth.host(run.tgt["pos0"]).astype(np.int64)
    ctx = synth.host(run.tgt["ctx_len"]).astype(np.int64)
    positions = (pos0[:, None] + np.arange(G)[None, :]).reshape(T)
    g = {k: f64(v) if v.dtype != torch.int32 else synth.host(v) for k, v in st.items()}

    if li == 0:
        assert np.array_equal(synth.host(st["x_in"]), synth.host(run.tgt["embeds"]).reshape(T, H))
    say(f"layer {li}: norm, kernel projection, conv prepare")
    assert_bf16_close(g["n"], O.rms_norm(g["x_in"], W("input_layernorm.weight"), d.rms_eps), "n")
    assert_bf16_close(g["coef"], O.linear(g["n"], W("attention_conv.kernel_projection.weight")), "kernel projection")
    base_a = O.as_f64(W("attention_conv.base_kernel"))
    assert_bf16_close(g["a"], _conv(g["n"], g["coef"][:, :2 * ng], base_a[0], d, G), "conv prepare")
    assert np.array_equal(synth.host(st["coef1"]), synth.host(st["coef"])[:, 2 * ng:]), "side-1 deltas"

    say(f"layer {li}: q|k|v + norm + RoPE, attention, o")
    a = g["a"][rows]
    q = O.rope_neox(O.rms_norm(O.linear(a, W("self_attn.q_proj.weight")).reshape(-1, NH, D),
                               W("self_attn.q_norm.weight"), d.rms_eps), positions[rows], d.rope_theta)
    k = O.rope_neox(O.rms_norm(O.linear(a, W("self_attn.k_proj.weight")).reshape(-1, NKV, D),
                               W("self_attn.k_norm.weight"), d.rms_eps), positions[rows], d.rope_theta)
    v = O.linear(a, W("self_attn.v_proj.weight"))
    want = np.concatenate([q.reshape(len(rows), -1), k.reshape(len(rows), -1), v], axis=1)
    assert_bf16_close(g["qkv"][rows], want, "q|k|v after norm and RoPE")
    window = O.layer_window(d, li)
    for b in reqs:
        r = slice(b * G, (b + 1) * G)
        qkv = g["qkv"][r]
        kc = synth.host(run.K[li][b:b + 1, :ctx[b]])
        vc = synth.host(run.V[li][b:b + 1, :ctx[b]])
        o = O.attention(qkv[:, :NH * D].reshape(1, G, NH, D), kc, vc,
                        qkv[:, NH * D:(NH + NKV) * D].reshape(1, G, NKV, D), qkv[:, (NH + NKV) * D:].reshape(1, G, NKV, D),
                        ctx[b:b + 1], pos0[b:b + 1], window)
        assert_bf16_close(g["attn"][r], o.reshape(G, NH * D), f"attention request {b}")
    assert_bf16_close(g["u"][rows], O.linear(g["attn"][rows], W("self_attn.o_proj.weight")), "o projection")

    say(f"layer {li}: conv finish + residual + norm, MLP")
    assert_bf16_close(g["x_mid"], g["x_in"] + _conv(g["u"], g["coef1"], base_a[1], d, G), "attention residual")
    assert_bf16_close(g["m"], O.rms_norm(g["x_mid"], W("post_attention_layernorm.weight"), d.rms_eps), "m")
    assert_bf16_close(g["coef_mlp"], O.linear(g["m"], W("mlp_conv.kernel_projection.weight")), "MLP kernel projection")
    base_m = O.as_f64(W("mlp_conv.base_kernel"))
    assert_bf16_close(g["i"], _conv(g["m"], g["coef_mlp"][:, :2 * ng], base_m[0], d, G), "MLP conv prepare")
    assert np.array_equal(synth.host(st["coef1_mlp"]), synth.host(st["coef_mlp"])[:, 2 * ng:]), "MLP side-1 deltas"
    i = g["i"][rows]
    gate = O.linear(i, W("mlp.gate_proj.weight"))
    up = O.linear(i, W("mlp.up_proj.weight"))
    assert_bf16_close(g["p"][rows], O.silu(gate) * up, "silu(gate) * up")
    assert_bf16_close(g["f"][rows], O.linear(g["p"][rows], W("mlp.down_proj.weight")), "down projection")
    assert_bf16_close(g["x_out"], g["x_mid"] + _conv(g["f"], g["coef1_mlp"], base_m[1], d, G), "MLP residual")
    if li + 1 < d.layers:
        gam = run.host_weight(f"layers.{li + 1}.input_layernorm.weight")
        assert_bf16_close(g["n_next"], O.rms_norm(g["x_out"], gam, d.rms_eps), "next layer's input norm")
    else:
        x = g["x_out"].reshape(Bq, G, H)[:, 1:, :].reshape(-1, H)
        assert_bf16_close(g["h"], O.rms_norm(x, run.host_weight("norm.weight"), d.rms_eps), "final norm, rows 1..G-1")


def check_tail(run, st, tokens, logits, max_rows=None):
    d, G, Bq = run.d, run.G, run.Bq
    N, K = Bq * (G - 1), d.top_k
    h = f64(st["h"])
    lg = synth.host(logits).reshape(N, d.vocab)
    assert np.isfinite(lg).all()
    say("tail: head logits on sampled columns, tile maxima")
    rng = np.random.default_rng(11)
    cand = synth.host(st["cand"])
    cols = np.unique(np.concatenate([rng.choice(d.vocab, min(d.vocab, 768), replace=False), [d.vocab - 1],
                                     cand.reshape(-1)]))
    head = run.tgt["lm_head"]
    w_cols = synth.host(head[torch.as_tensor(cols, device=DEV)])
    assert_bf16_close(lg[:, cols], O.head_logits(h, w_cols), "head logits (sampled columns)")
    ntiles = (d.vocab + 255) // 256
    pad = np.full((N, ntiles * 256), -np.inf, dtype=np.float32)
    pad[:, :d.vocab] = lg
    assert np.array_equal(synth.host(st["tile_max"]), pad.reshape(N, ntiles, 256).max(axis=-1)), "tile maxima"
    say("tail: candidates, selector projection, score_edges, walk")
    sel = np.arange(N) if max_rows is None or N <= max_rows else np.linspace(0, N - 1, max_rows).astype(int)
    want_ids, want_un = O.compute_candidates(lg[sel], K)
    assert np.array_equal(cand[sel], want_ids), "candidate ids"
    assert np.array_equal(synth.host(st["unary"])[sel], want_un), "candidate logits"
    z = f64(st["z"])
    assert_bf16_close(z, O.selector_project(h, run.host_weight("candidate_selector.hidden_projection.weight")),
                      "selector projection")
    S = G - 1
    want_sc = O.score_edges(cand.reshape(Bq, S, K), synth.host(st["unary"]).reshape(Bq, S, K).astype(np.float64),
                            z.reshape(Bq, S, -1), synth.host(run.tgt["anchors"]),
                            run.host_weight("candidate_selector.predecessor_codebook"),
                            run.host_weight("candidate_selector.successor_codebook"))
    sc = synth.host(st["scores"]).reshape(Bq, S, K, K)
    assert_f32_close(sc, want_sc, "score_edges given the GPU's candidates and z")
    assert np.array_equal(synth.host(tokens), O.select_path(sc, cand.reshape(Bq, S, K))), "walk over the GPU's scores"


def _stages(name, layer):
    run = _run(name)
    say(f"{name}: traced draft block, layer {layer}")
    st, tokens, logits = run.traced(layer)
    check_layer(run, layer, st)
    check_tail(run, st, tokens, logits, max_rows=96)


@pytest.mark.parametrize("name,layer", [("tiny3", 0), ("tiny_sw", 0), ("tiny_sw", 1), ("full", 0), ("full", 4)])
def test_draft_stages_match_oracle(name, layer):
    _stages(name, layer)


def test_context_stages_match_oracle():
    """fc, hidden norm, one layer's k|v projection and the K/V store at the full workload's
    context (B=8, L=2048), on sampled rows."""
    w = configs.FULL
    d = w.dims
    run = _run("full")
    Bq, L, H = w.batch, w.ctx_len, d.hidden
    M, kvw = Bq * L, 2 * d.kv_heads * d.head_dim
    NKV, D = d.kv_heads, d.head_dim
    li = 3
    tgt = run.tgt
    st = {"fc_out": torch.full((M, H), float("nan"), dtype=torch.bfloat16, device=DEV),
          "c": torch.full((M, H), float("nan"), dtype=torch.bfloat16, device=DEV),
          "kv": torch.full((M, kvw), float("nan"), dtype=torch.bfloat16, device=DEV)}
    K, V = run.dr.alloc_kv(Bq, L)
    ws = B_.workspace(B_.dfl_context_workspace_bytes(run.dr.handle, Bq, L))
    B_.dfl_context_materialize_traced(run.dr.handle, tgt["taps"], Bq, L, 0, L, K, V, ws, li, st)
    torch.cuda.synchronize()
    for i in range(d.layers):   # the traced call materialises what the plain one does
        assert torch.equal(K[i], run.K[i]) and torch.equal(V[i], run.V[i])
    rows = np.concatenate([np.arange(0, 48), np.arange(M - 48, M), 5 * L + np.arange(100, 132)])
    say("context: fc on sampled rows, hidden norm on all rows")
    taps = f64(tgt["taps"].reshape(M, -1)[torch.as_tensor(rows, device=DEV)])
    assert_bf16_close(f64(st["fc_out"])[rows], O.linear(taps, run.host_weight("fc.weight")), "fc")
    fc = f64(st["fc_out"])
    cc = f64(st["c"])
    assert_bf16_close(cc, O.rms_norm(fc, run.host_weight("hidden_norm.weight"), d.rms_eps), "hidden norm")
    p = f"layers.{li}."
    wkv = np.concatenate([run.host_weight(p + "self_attn.k_proj.weight"), run.host_weight(p + "self_attn.v_proj.weight")])
    kv = f64(st["kv"])
    assert_bf16_close(kv[rows], O.linear(cc[rows], wkv), "context k|v projection")
    say("context: K store (k_norm + RoPE at the row's position), V copy")
    pos = rows % L
    want_k = O.rope_neox(O.rms_norm(kv[rows, :NKV * D].reshape(-1, NKV, D), run.host_weight(p + "self_attn.k_norm.weight"),
                                    d.rms_eps), pos, d.rope_theta)
    got_k = f64(K[li].reshape(M, NKV, D)[torch.as_tensor(rows, device=DEV)])
    assert_bf16_close(got_k, want_k, "K store")
    got_v = synth.host(V[li].reshape(M, NKV * D)[torch.as_tensor(rows, device=DEV)])
    assert np.array_equal(got_v, synth.host(st["kv"])[rows, NKV * D:]), "V store"


def test_ragged_append_stages_match_oracle():
    """The ragged append's K/V store at the full drafter's shapes: three requests append 5,
    0 and 300 rows at their own positions; every written row matches k_norm + RoPE of the
    traced k|v rows at its position, V is the traced v rows, and no other row is touched."""
    run = _run("full")
    d = run.d
    H, NKV, D = d.hidden, d.kv_heads, d.head_dim
    counts, starts = [5, 0, 300], [10, 0, 1500]
    offsets = np.concatenate([[0], np.cumsum(counts)]).tolist()
    rows = offsets[-1]
    Lcap, li = 2048, 2
    taps = synth.normal((rows, d.n_taps * H), 0.0, 1.0, seed=91, device=DEV)
    K, V = run.dr.alloc_kv(3, Lcap)
    st = {"kv": torch.full((rows, 2 * NKV * D), float("nan"), dtype=torch.bfloat16, device=DEV)}
    ws = B_.workspace(B_.dfl_context_append_workspace_bytes(run.dr.handle, 3, rows))
    B_.dfl_context_append_traced(run.dr.handle, taps, offsets, starts, 3, Lcap, K, V, ws, li, st)
    torch.cuda.synchronize()
    kv = f64(st["kv"])
    p = f"layers.{li}."
    for b in range(3):
        n, s0 = counts[b], starts[b]
        kb, vb = f64(K[li][b]), synth.host(V[li][b])
        outside = np.ones(Lcap, dtype=bool)
        outside[s0:s0 + n] = False
        assert not kb[outside].any() and not vb[outside].any(), f"request {b}: rows outside were written"
        if n == 0:
            continue
        src = kv[offsets[b]:offsets[b + 1]]
        want = O.rope_neox(O.rms_norm(src[:, :NKV * D].reshape(n, NKV, D), run.host_weight(p + "self_attn.k_norm.weight"),
                                      d.rms_eps), s0 + np.arange(n), d.rope_theta)
        assert_bf16_close(kb[s0:s0 + n], want, f"request {b} K store")
        assert np.array_equal(vb[s0:s0 + n].reshape(n, -1), synth.host(st["kv"])[offsets[b]:offsets[b + 1], NKV * D:])


def test_long_draft_stages_match_oracle():
    """64 requests (T = 1024 block rows, 960 head rows) over 8192 given context rows: the
    projections run on the 256 x 256 tiles, the head on them with the tile-maxima epilogue."""
    _stages("long", 4)
