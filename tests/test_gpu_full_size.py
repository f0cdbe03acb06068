"""Parity at the full workload sizes, in the launch configuration bench.py times.

The oracle recomputes request 0 of each batch from its own inputs (requests are
independent, so request 0 of the batched launch must equal the oracle's single-request
result); every request is also checked against properties that hold at any size.
"""
import numpy as np
import pytest
import torch

from dflash2_block_drafter_amd import binding as B
from dflash2_block_drafter_amd import configs, synth
from dflash2_block_drafter_amd.drafter import Drafter
from oracle import dflash2 as O
from tests.helpers import assert_composed_close, assert_f32_close, assert_layer_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(f"[full-size] {msg}", flush=True)


def _drafted_tokens_are_topk(tokens, logits, K):
    """Every drafted token is one of the K best logits of its slot (a property of the walk)."""
    lg = logits.reshape(-1, logits.shape[-1])
    tk = tokens.reshape(-1)
    kth = -np.partition(-lg, K - 1, axis=1)[:, K - 1]
    chosen = lg[np.arange(lg.shape[0]), tk]
    assert np.all(chosen >= kth), "a drafted token is not among its slot's top-K logits"


def _host_weights(weights, layers=None):
    return {k: synth.host(v) for k, v in weights.items()}


def _layer_parity(w, layer_ids, sample):
    """One layer at a time, from the same synthetic bf16 block rows and context K/V on both
    sides, in the batch the benchmark launches; the oracle computes the sampled requests."""
    d = w.dims
    Bq, G, L = w.batch, d.block_size, w.ctx_len
    say(f"{w.name}: weights on the GPU, B={Bq} G={G} L={L}")
    weights = synth.drafter_weights(w, device=DEV)
    dr = Drafter(d, weights)
    wh = _host_weights(weights)
    x = synth.normal((Bq * G, d.hidden), 0.0, 1.0, seed=synth.seed_for(w.seed, "layer-test.x"), device=DEV)
    ctx_len = torch.full((Bq,), L, dtype=torch.int32, device=DEV)
    pos0 = torch.full((Bq,), L, dtype=torch.int32, device=DEV)
    ws = dr.workspace(Bq, G, L)
    xh = O.as_f64(synth.host(x)).reshape(Bq, G, d.hidden)
    worst = 0.0
    for li in layer_ids:
        k, v = synth.given_kv(w, li, device=DEV)
        y = torch.empty_like(x)
        say(f"layer {li}: GPU")
        B.dfl_block_layer(dr.handle, li, x, y, Bq, G, k, v, L, L, ctx_len, pos0, ws)
        torch.cuda.synchronize()
        yg = synth.host(y).reshape(Bq, G, d.hidden)
        lw = O.layer_weights(wh, li)
        for b in sample:
            kb, vb = synth.host(k[b:b + 1]), synth.host(v[b:b + 1])
            ctx = np.array([L])
            ref = O.block_layer(xh[b:b + 1], lw, kb, vb, ctx, ctx, d, bf16_points=True)
            ref64 = O.block_layer(xh[b:b + 1], lw, kb, vb, ctx, ctx, d)
            got = O.as_f64(yg[b:b + 1])
            rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
            scale = np.abs(ref) + rms
            gpu_err = np.abs(got - ref) / scale
            spread = np.abs(ref64 - ref) / scale
            say(f"layer {li} request {b}: GPU vs oracle max {gpu_err.max():.3g} mean {gpu_err.mean():.3g}; "
                f"oracle fp64 vs bf16 points max {spread.max():.3g} mean {spread.mean():.3g}")
            worst = max(worst, gpu_err.max())
            assert_layer_close(got, ref, ref64, f"layer {li} output, request {b}")
    dr.close()
    return worst


def test_full_drafter_layers_match_oracle():
    _layer_parity(configs.FULL, range(configs.FULL.dims.layers), sample=(0, configs.FULL.batch - 1))


def test_long_context_layer_matches_oracle():
    _layer_parity(configs.LONG, [0], sample=(0, configs.LONG.batch - 1))


def test_full_drafter_end_to_end_properties():
    """The full draft block in the bench's launch configuration: every drafted token is a
    valid id among its slot's top-K head logits, two runs agree bit for bit, and a run with
    the target head bound (tile-contiguous copy) agrees with them bit for bit."""
    w = configs.FULL
    d = w.dims
    say("full drafter end to end (B=8, L=2048)")
    weights = synth.drafter_weights(w, device=DEV)
    tgt = synth.target_inputs(w, device=DEV)
    dr = Drafter(d, weights)
    K, V = dr.alloc_kv(w.batch, w.ctx_len)
    dr.materialize(tgt["taps"], K, V)
    outs = []
    for _ in range(2):
        outs.append(dr.draft(tgt["embeds"], tgt["anchors"], K, V, w.ctx_len, tgt["ctx_len"], tgt["pos0"],
                             tgt["lm_head"], want_logits=True))
    torch.cuda.synchronize()
    dr.bind_target(tgt["lm_head"])   # the bench's setup: the head streamed from the bound copy
    outs.append(dr.draft(tgt["embeds"], tgt["anchors"], K, V, w.ctx_len, tgt["ctx_len"], tgt["pos0"],
                         None, want_logits=True))
    torch.cuda.synchronize()
    (t1, l1), (t2, l2), (t3, l3) = outs
    assert torch.equal(t1, t2) and torch.equal(l1, l2)
    assert torch.equal(t1, t3) and torch.equal(l1, l3), "bound head must match the borrowed one bit for bit"
    tok, lg = t1.cpu().numpy(), l1.cpu().numpy()
    assert tok.min() >= 0 and tok.max() < d.vocab
    _drafted_tokens_are_topk(tok, lg, d.top_k)
    dr.close()


@pytest.mark.parametrize("w", [configs.FULL, configs.LONG], ids=["full", "long"])
def test_draft_without_logits_matches_with_logits(w):
    """Without a logits output the head stores only the logit tiles that can hold one of a
    row's top 16 (by the bound its workgroups build up) and the top-K reads only those; the
    tokens must be the ones drafted when every logit is stored, and each among its slot's
    top-K logits."""
    d = w.dims
    say(f"{w.name}: draft with and without logits, B={w.batch} L={w.ctx_len}")
    weights = synth.drafter_weights(w, device=DEV)
    tgt = synth.target_inputs(w, device=DEV, with_taps=not w.kv_given)
    dr = Drafter(d, weights)
    if w.kv_given:
        K, V = map(list, zip(*(synth.given_kv(w, i, device=DEV) for i in range(d.layers))))
    else:
        K, V = dr.alloc_kv(w.batch, w.ctx_len)
        dr.materialize(tgt["taps"], K, V)
    dr.bind_target(tgt["lm_head"])
    args = (tgt["embeds"], tgt["anchors"], K, V, w.ctx_len, tgt["ctx_len"], tgt["pos0"], None)
    t_full, lg = dr.draft(*args, want_logits=True)
    t_a = dr.draft(*args).clone()
    t_b = dr.draft(*args).clone()   # the workspace now holds the previous block's logits
    torch.cuda.synchronize()
    assert torch.equal(t_a, t_full), "tokens differ when the head skips tiles"
    assert torch.equal(t_b, t_full)
    _drafted_tokens_are_topk(t_full.cpu().numpy(), lg.cpu().numpy(), d.top_k)
    dr.close()


def test_head_projection_full_size_sampled_columns():
    """The head GEMM at its full size (M = B*(G-1) = 120, V = 248320, H = 5120), row-major
    weight as the target lends it; the oracle computes 512 sampled vocabulary columns."""
    M, N, K = 120, 248320, 5120
    h = synth.normal((M, K), 0.0, 1.0, seed=701, device=DEV)
    W = synth.normal((N, K), 0.0, 0.02, seed=702, device=DEV)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    ws = B.workspace(B.dfl_linear_workspace_bytes(M, N, K))
    B.dfl_linear(h, M, K, K, W, N, y, N, 1, ws)
    torch.cuda.synchronize()
    cols = np.sort(np.random.default_rng(7).choice(N, 512, replace=False))
    cols[-1] = N - 1
    want = O.linear(synth.host(h), synth.host(W)[cols])
    from tests.helpers import assert_bf16_close
    assert_bf16_close(y[:, torch.as_tensor(cols, device=DEV)], want, "head columns")


def test_selector_microbench_full_size():
    cfg = configs.SELECTOR_BENCH
    Bq, S, H, K, V, R = cfg["B"], cfg["S"], cfg["hidden"], cfg["top_k"], cfg["vocab"], cfg["rank"]
    say("selector microbench B=32 S=15 V=248320 (stress codebooks N(0,0.5))")
    inp = synth.selector_inputs(Bq, S, H, K, V, R, cfg["seed"], device=DEV, book_std=0.5)
    N = Bq * S
    ids = torch.empty((Bq, S, K), dtype=torch.int32, device=DEV)
    unary = torch.empty((Bq, S, K), dtype=torch.float32, device=DEV)
    ws = B.workspace(B.dfl_candidates_workspace_bytes(N, V, K))
    B.dfl_compute_candidates(inp["logits"], N, V, K, ids, unary, ws)
    z = torch.empty((Bq, S, R), dtype=torch.float32, device=DEV)
    zws = B.workspace(B.dfl_selector_project_workspace_bytes(N, H, R))
    B.dfl_selector_project(inp["hidden"], N, H, inp["proj"], R, z, zws)
    scores = torch.empty((Bq, S, K, K), dtype=torch.float32, device=DEV)
    B.dfl_score_edges(ids, unary, z, inp["anchors"], Bq, S, K, R, inp["pred"], inp["succ"], V, scores)
    tokens = torch.empty((Bq, S), dtype=torch.int32, device=DEV)
    B.dfl_select_path(scores, ids, Bq, S, K, tokens)
    torch.cuda.synchronize()
    lg = inp["logits"].cpu().numpy()
    gid, gun = ids.cpu().numpy(), unary.cpu().numpy()
    flat = lg.reshape(N, V)
    say("oracle candidates for all 480 rows")
    want_ids, want_un = O.compute_candidates(flat, K)
    assert np.array_equal(gid.reshape(N, K), want_ids)
    assert np.array_equal(gun.reshape(N, K), want_un)
    want_z = O.selector_project(synth.host(inp["hidden"]).reshape(N, H), synth.host(inp["proj"]))
    assert_composed_close(z.reshape(N, R), want_z, "selector projection")
    want_sc = O.score_edges(want_ids.reshape(Bq, S, K), want_un.reshape(Bq, S, K), want_z.reshape(Bq, S, R),
                            inp["anchors"].cpu().numpy(), synth.host(inp["pred"]), synth.host(inp["succ"]))
    assert_f32_close(scores, want_sc, "score_edges on the GPU's own z", rel=1e-4)
    # score_edges given z: the oracle's candidates and z (as fp32) fed to both sides
    oz = torch.as_tensor(want_z.reshape(Bq, S, R).astype(np.float32), device=DEV)
    oc = torch.as_tensor(want_ids.reshape(Bq, S, K), device=DEV)
    ou = torch.as_tensor(want_un.reshape(Bq, S, K), device=DEV)
    sc2 = torch.empty_like(scores)
    B.dfl_score_edges(oc, ou, oz, inp["anchors"], Bq, S, K, R, inp["pred"], inp["succ"], V, sc2)
    torch.cuda.synchronize()
    want_sc2 = O.score_edges(want_ids.reshape(Bq, S, K), want_un.reshape(Bq, S, K),
                             oz.cpu().numpy().astype(np.float64), inp["anchors"].cpu().numpy(),
                             synth.host(inp["pred"]), synth.host(inp["succ"]))
    assert_f32_close(sc2, want_sc2, "score_edges given z at full size")
    # the walk, fed the oracle's fp32 scores, must give the oracle's tokens bit for bit
    osc = torch.as_tensor(want_sc.astype(np.float32), device=DEV)
    t2 = torch.empty((Bq, S), dtype=torch.int32, device=DEV)
    B.dfl_select_path(osc, ids, Bq, S, K, t2)
    torch.cuda.synchronize()
    assert np.array_equal(t2.cpu().numpy(), O.select_path(want_sc.astype(np.float32), want_ids.reshape(Bq, S, K)))
