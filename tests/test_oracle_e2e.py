"""End-to-end pins of the oracle's composition on the tiny drafter.

The pages print no worked values for a whole block, so parity of the composed
path with the authors' implementation is unpinned; these tests pin the
composition itself through special cases with closed forms and through the
request-independence the path has by construction.
"""
import numpy as np
import pytest
import torch

from dflash2_block_drafter_amd import configs, synth
from oracle import dflash2 as O


def _host(d):
    return {k: synth.host(v) for k, v in d.items()}


@pytest.fixture(scope="module")
def tiny():
    w = configs.TINY
    weights = _host(synth.drafter_weights(w))
    tgt = _host(synth.target_inputs(w))
    return w, weights, tgt


def test_context_row_zero_has_no_rotation(tiny):
    # position 0 leaves K unrotated: K[b, 0] = k_norm(k_proj c_0)   (dflash2.ts #contextKV)
    w, weights, tgt = tiny
    d = w.dims
    c = O.project_context(tgt["taps"], weights["fc.weight"], weights["hidden_norm.weight"], d.rms_eps)
    ks, vs = O.materialize_context(tgt["taps"], weights, d)
    k0 = O.rms_norm((c[:, 0] @ O.as_f64(weights["layers.0.self_attn.k_proj.weight"]).T)
                    .reshape(w.batch, d.kv_heads, d.head_dim),
                    weights["layers.0.self_attn.k_norm.weight"], d.rms_eps)
    assert np.allclose(ks[0][:, 0], k0, rtol=1e-12)
    assert np.allclose(vs[0], (c @ O.as_f64(weights["layers.0.self_attn.v_proj.weight"]).T)
                       .reshape(vs[0].shape), rtol=1e-12)


def test_zero_sublayers_reduce_to_argmax_of_head(tiny):
    # With every projection inside the layers zeroed, both sublayer outputs are zero, so
    # x passes through unchanged; with zero codebooks the walk is argmax decoding.  All
    # mask rows carry the same embedded token, so every slot drafts
    # argmax_v <norm(mask_row), lm_head[v]>.
    w, weights, tgt = tiny
    d = w.dims
    wz = dict(weights)
    for name in list(wz):
        if name.startswith("layers.") and name.endswith("_proj.weight"):
            wz[name] = np.zeros_like(wz[name])
    for name in ("candidate_selector.predecessor_codebook", "candidate_selector.successor_codebook"):
        wz[name] = np.zeros_like(wz[name])
    ks, vs = O.materialize_context(tgt["taps"], wz, d)
    tokens = O.draft_block(tgt["embeds"], wz, tgt["lm_head"], tgt["anchors"], ks, vs,
                           tgt["ctx_len"], tgt["pos0"], d)
    mask_row = O.as_f64(tgt["embeds"])[0, 1]
    g = O.as_f64(weights["norm.weight"])
    h = mask_row / np.sqrt(np.mean(mask_row ** 2) + d.rms_eps) * g
    want = int(np.argmax((h @ O.as_f64(tgt["lm_head"]).T).astype(np.float32)))
    assert np.all(tokens == want)


def test_requests_are_independent():
    # Every step is per request except the shared weights: drafting two requests
    # together gives each the tokens it gets alone.
    w2 = configs.with_batch(configs.TINY, 2)
    d = w2.dims
    weights = _host(synth.drafter_weights(w2))
    tgt = _host(synth.target_inputs(w2))
    ks, vs = O.materialize_context(tgt["taps"], weights, d)
    both = O.draft_block(tgt["embeds"], weights, tgt["lm_head"], tgt["anchors"], ks, vs,
                         tgt["ctx_len"], tgt["pos0"], d, return_all=True)
    for b in range(2):
        one = O.draft_block(tgt["embeds"][b:b + 1], weights, tgt["lm_head"], tgt["anchors"][b:b + 1],
                            [k[b:b + 1] for k in ks], [v[b:b + 1] for v in vs],
                            tgt["ctx_len"][b:b + 1], tgt["pos0"][b:b + 1], d, return_all=True)
        assert np.allclose(one["h"][0], both["h"][b], rtol=1e-12, atol=1e-12)
        assert np.array_equal(one["tokens"][0], both["tokens"][b])


def test_bf16_points_stay_close(tiny):
    # Rounding activations where the dflash2.ts #block casts to bf16 moves the final
    # hidden rows by far less than the bf16-in/fp32-accumulate tolerance.
    w, weights, tgt = tiny
    d = w.dims
    ks, vs = O.materialize_context(tgt["taps"], weights, d)
    h = O.draft_hidden(tgt["embeds"], weights, ks, vs, tgt["ctx_len"], tgt["pos0"], d)
    hr = O.draft_hidden(tgt["embeds"], weights, ks, vs, tgt["ctx_len"], tgt["pos0"], d, bf16_points=True)
    assert np.all(np.abs(hr - h) <= 2e-3 + 2e-2 * np.abs(h))
    assert not np.array_equal(hr, h)


def test_draft_vocabulary_reduces_to_masked_full_head(tiny):
    """A draft vocabulary listing every id in order is the plain path; an ascending subset
    gives exactly the top-K of the full head's logits with the unlisted columns at -inf
    (the plain top-k routine, pinned by brute force), mapped to token ids."""
    w, weights, tgt = tiny
    d = w.dims
    ks, vs = O.materialize_context(tgt["taps"], weights, d)
    args = (tgt["embeds"], weights, tgt["lm_head"], tgt["anchors"], ks, vs, tgt["ctx_len"], tgt["pos0"], d)
    full = O.draft_block(*args, return_all=True)
    same = O.draft_block(*args, return_all=True, vocab_ids=np.arange(d.vocab))
    assert np.array_equal(full["tokens"], same["tokens"]) and np.array_equal(full["logits"], same["logits"])
    rng = np.random.default_rng(12)
    ids = np.sort(rng.choice(d.vocab, size=300, replace=False))
    sub = O.draft_block(*args, return_all=True, vocab_ids=ids)
    masked = np.full_like(full["logits"], -np.inf)
    masked[..., ids] = full["logits"][..., ids]
    cand, unary = O.compute_candidates(masked, d.top_k)
    assert np.array_equal(sub["cand"], cand) and np.array_equal(sub["unary"], unary)
    assert np.array_equal(sub["logits"], full["logits"][..., ids])
    assert np.isin(sub["tokens"], ids).all()
