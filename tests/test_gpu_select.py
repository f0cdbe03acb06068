"""The two-launch selection (top-k from tile maxima or from its own scan of the logits, then
score_edges and the walk) against the three single-step calls and against the oracle:
candidates and their logits bit for bit, scores at the fp32 bar, tokens bit for bit given
the scores."""
import numpy as np
import pytest
import torch

from dflash2_block_drafter_amd import binding as B
from dflash2_block_drafter_amd import synth
from oracle import dflash2 as O
from tests.helpers import assert_f32_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(Bq, S, V, K, R, kind, seed):
    logits = synth.normal((Bq * S, V), 0.0, 3.0, seed=seed, device=DEV, dtype=torch.float32)
    if kind == "ties":            # a quarter of the row on one value above the rest: many tiles reach theta
        logits[:, ::4] = 9.5
    elif kind == "constant":      # every value ties: the merging scan over every tile
        logits[:] = 1.25
    elif kind == "few_hot":       # K hot values in one tile, the rest low
        logits[:] = -5.0
        logits[:, 300:300 + K] = torch.arange(K, device=DEV, dtype=torch.float32)
    elif kind == "hot_ties":      # 80 equal maxima in 80 tiles: more than 64 values reach theta
        logits[:, 1000:1000 + 3001 * 80:3001] = 20.0
    elif kind == "negative":      # every logit far below zero, tile maxima not integers
        logits -= 50.0
    elif kind == "neg_inf":       # mostly -inf, a finite value every 997 columns
        finite = logits[:, ::997].clone()
        logits[:] = float("-inf")
        logits[:, ::997] = finite
    z = synth.normal((Bq * S, R), 0.0, 1.0, seed=seed + 1, device=DEV, dtype=torch.float32)
    pred = synth.normal((V, R), 0.0, 0.5, seed=seed + 2, device=DEV)
    succ = synth.normal((V, R), 0.0, 0.5, seed=seed + 3, device=DEV)
    anchors = synth.uniform_ids(Bq, V, seed=seed + 4, device=DEV)
    return logits, z, pred, succ, anchors


@pytest.mark.parametrize("Bq,S,V,K,R,kind", [
    (32, 15, 248320, 16, 64, "normal"),   # the selector workload, stress codebooks
    (8, 15, 248320, 16, 64, "ties"),
    (3, 7, 1024, 4, 16, "normal"),        # the tiny drafter's selector
    (2, 5, 10001, 8, 32, "normal"),       # a ragged last tile
    (2, 6, 5000, 16, 64, "constant"),
    (3, 4, 20000, 16, 64, "few_hot"),
    (4, 1, 3000, 2, 8, "normal"),         # one slot
    (1, 63, 4096, 16, 64, "normal"),      # more slots than wavefronts
    (2, 3, 248320, 16, 64, "hot_ties"),
    (2, 5, 70000, 16, 64, "neg_inf"),
    (4, 15, 248320, 16, 64, "negative"),
])
def test_select_tokens_matches_steps_and_oracle(Bq, S, V, K, R, kind):
    print(f"[select] B={Bq} S={S} V={V} K={K} R={R} {kind}", flush=True)
    N = Bq * S
    logits, z, pred, succ, anchors = _inputs(Bq, S, V, K, R, kind, seed=900 + V % 97)
    tmax = torch.empty((N, (V + 255) // 256), dtype=torch.float32, device=DEV)
    B.dfl_tile_maxima(logits, N, V, tmax)
    cand = torch.full((N, K), -1, dtype=torch.int32, device=DEV)
    unary = torch.full((N, K), float("nan"), dtype=torch.float32, device=DEV)
    scores = torch.full((N, K, K), float("nan"), dtype=torch.float32, device=DEV)
    tokens = torch.full((Bq, S), -1, dtype=torch.int32, device=DEV)
    B.dfl_select_tokens(logits, tmax, Bq, S, V, K, z, R, anchors, pred, succ, cand, unary, scores, tokens)
    # the single-step calls
    c2 = torch.empty_like(cand)
    u2 = torch.empty_like(unary)
    ws = B.workspace(B.dfl_candidates_workspace_bytes(N, V, K))
    B.dfl_compute_candidates(logits, N, V, K, c2, u2, ws)
    s2 = torch.empty_like(scores)
    B.dfl_score_edges(c2, u2, z, anchors, Bq, S, K, R, pred, succ, V, s2)
    t2 = torch.empty_like(tokens)
    B.dfl_select_path(s2, c2, Bq, S, K, t2)
    # without tile maxima: one workgroup per row scans its logits, then takes its top-k
    c3 = torch.full_like(cand, -1)
    u3 = torch.full_like(unary, float("nan"))
    s3 = torch.full_like(scores, float("nan"))
    t3 = torch.full_like(tokens, -1)
    B.dfl_select_tokens(logits, None, Bq, S, V, K, z, R, anchors, pred, succ, c3, u3, s3, t3)
    torch.cuda.synchronize()
    assert torch.equal(cand, c2) and torch.equal(unary, u2)
    assert torch.equal(scores, s2), "edge scores differ from dfl_score_edges"
    assert torch.equal(tokens, t2)
    assert torch.equal(cand, c3) and torch.equal(unary, u3), "the scanning top-k differs"
    assert torch.equal(scores, s3) and torch.equal(tokens, t3)
    # with the projection in the scan's launch: the same z as dfl_selector_project, and the
    # same selection as dfl_select_tokens given that z
    H = 5120 if V > 100000 else 256
    hid = synth.normal((N, H), 0.0, 1.0, seed=950 + V % 89, device=DEV)
    proj = synth.normal((R, H), 0.0, 0.02, seed=951 + V % 89, device=DEV)
    zp = torch.full((N, R), float("nan"), dtype=torch.float32, device=DEV)
    c4, u4, s4, t4 = (torch.full_like(cand, -1), torch.full_like(unary, float("nan")),
                      torch.full_like(scores, float("nan")), torch.full_like(tokens, -1))
    B.dfl_select_tokens_projected(logits, Bq, S, V, K, hid, H, proj, R, zp, anchors, pred, succ, c4, u4, s4, t4)
    zr = torch.empty_like(zp)
    B.dfl_selector_project(hid, N, H, proj, R, zr, None)
    c5, u5, s5, t5 = (torch.empty_like(cand), torch.empty_like(unary), torch.empty_like(scores),
                      torch.empty_like(tokens))
    B.dfl_select_tokens(logits, None, Bq, S, V, K, zr, R, anchors, pred, succ, c5, u5, s5, t5)
    torch.cuda.synchronize()
    assert torch.equal(zp, zr), "the projection in the scan's launch differs from dfl_selector_project"
    assert torch.equal(c4, cand) and torch.equal(u4, unary)
    assert torch.equal(s4, s5) and torch.equal(t4, t5)
    # the oracle
    lg = logits.cpu().numpy()
    rows = np.arange(N) if N <= 96 else np.linspace(0, N - 1, 96).astype(int)
    want_ids, want_un = O.compute_candidates(lg[rows], K)
    assert np.array_equal(cand.cpu().numpy()[rows], want_ids)
    assert np.array_equal(unary.cpu().numpy()[rows], want_un)
    want_sc = O.score_edges(cand.cpu().numpy().reshape(Bq, S, K), unary.cpu().numpy().reshape(Bq, S, K).astype(np.float64),
                            z.cpu().numpy().reshape(Bq, S, R).astype(np.float64), anchors.cpu().numpy(),
                            synth.host(pred), synth.host(succ))
    sc = scores.cpu().numpy().reshape(Bq, S, K, K)
    assert_f32_close(sc, want_sc, "edge scores")
    assert np.array_equal(tokens.cpu().numpy(), O.select_path(sc, cand.cpu().numpy().reshape(Bq, S, K)))
