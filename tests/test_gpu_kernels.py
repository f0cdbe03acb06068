"""Per-step parity of the HIP kernels against the CPU oracle, through the C ABI.

Sizes span several tiles and a ragged tail; the oracle computes in float64 from the same
bf16 bits.  Top-k ids and select_path tokens are compared bit for bit.
"""
import numpy as np
import pytest
import torch

from dflash2_block_drafter_amd import binding as B
from dflash2_block_drafter_amd import synth
from oracle import dflash2 as O
from tests.helpers import assert_bf16_close, assert_f32_close

pytestmark = pytest.mark.gpu
DEV = "cuda"


def bf(shape, seed, mean=0.0, std=1.0):
    return synth.normal(shape, mean, std, seed=seed, device=DEV)


def h(t):
    return synth.host(t)


@pytest.mark.parametrize("M,N,K,out_f32", [
    (40, 200, 320, False),      # ragged M and N, one K tile pair
    (300, 256, 512, True),      # several M tiles, ragged M
    (128, 1280, 5120, True),    # split-K path (kernel_projection shape)
    (128, 4096, 1024, False),
    (120, 1000, 256, True),     # N not a multiple of 64
    (9, 640, 1024, False),      # one 16-row fragment, split K
    (20, 384, 512, True),       # two 16-row fragments
    # wide projections (N >= 16384, >= 64M weights) take the weight-streaming kernel: 1, 2, 4
    # and 8 row fragments
    (9, 16384, 4096, False),
    (30, 16640, 4096, True),    # N not a multiple of the 256-column workgroup
    (50, 32768, 2048, False),
    (128, 16384, 4096, True),
    (100, 16500, 4096, False),  # the last 160-row workgroup partly past N
    # deep projections at M <= 128: five wavefronts, K split 8 (the down projection's plan)
    (128, 5120, 17408, False),
    (70, 4960, 12800, True),    # N not a multiple of 160, ragged M
    # mid-size projections at M <= 128: two wavefronts, K split to fill a round (o's plan)
    (128, 5120, 4096, False),
    (120, 4950, 4096, True),    # N not a multiple of 64
    # 256 x 256 workgroup tiles once they fill a round of 256 workgroups
    (512, 32768, 256, False),
    (300, 32868, 320, True),    # ragged M and N
    # 256 x 256 tiles with split K when they do not fill a round (o / down at 64 requests)
    (600, 4096, 1024, True),
    (520, 5000, 2048, False),   # ragged M and N, bf16 out through the split-K reduce
    # a last round of 256 x 256 tiles at most half full: its weight rows run split K
    (512, 33024, 1024, True),
    (300, 65792, 1024, False),
])
def test_linear(M, N, K, out_f32):
    x = bf((M, K), 11)
    w = bf((N, K), 12, std=0.02)
    y = torch.empty((M, N), dtype=torch.float32 if out_f32 else torch.bfloat16, device=DEV)
    ws = B.workspace(B.dfl_linear_workspace_bytes(M, N, K))
    B.dfl_linear(x, M, K, K, w, N, y, N, out_f32, ws)
    torch.cuda.synchronize()
    want = O.linear(h(x), h(w))
    assert_bf16_close(y, want, f"linear {M}x{N}x{K}")
    if out_f32:
        # only the accumulation order differs from the float64 result
        assert_f32_close(y, want, "linear fp32 accumulation", rel=1e-4)


@pytest.mark.parametrize("rows,H", [(37, 5120), (8, 256), (130, 1024)])
def test_rms_norm(rows, H):
    x = bf((rows, H), 21)
    g = bf((H,), 22, 1.0, 0.02)
    y = torch.empty_like(x)
    B.dfl_rms_norm(x, rows, H, H, g, 1e-6, y, H)
    torch.cuda.synchronize()
    assert_bf16_close(y, O.rms_norm(h(x), h(g), 1e-6), "rms_norm")


@pytest.mark.parametrize("D,heads,G", [(128, 10, 16), (64, 6, 8)])
def test_head_norm_rope(D, heads, G):
    Bq = 3
    rows = Bq * G
    x = bf((rows, heads * D + 64), 31)      # leading dimension wider than the heads
    g = bf((D,), 32, 1.0, 0.02)
    pos0 = torch.tensor([0, 2048, 8192], dtype=torch.int32, device=DEV)
    ref = h(x)
    B.dfl_head_norm_rope(x, rows, heads, D, heads * D + 64, g, 1e-6, 1e7, pos0, G)
    torch.cuda.synchronize()
    xin = O.as_f64(ref)[:, :heads * D].reshape(rows, heads, D)
    pos = (np.array([0, 2048, 8192])[:, None] + np.arange(G)[None, :]).reshape(rows)
    want = O.rope_neox(O.rms_norm(xin, h(g), 1e-6), pos, 1e7)
    assert_bf16_close(x[:, :heads * D].reshape(rows, heads, D), want, "head_norm_rope")
    assert np.array_equal(h(x)[:, heads * D:], ref[:, heads * D:]), "columns past the heads changed"


@pytest.mark.parametrize("D,NH,NKV,G,ctx", [
    (128, 8, 2, 16, [600, 0, 257]),   # several 64-key tiles and chunks, empty and ragged contexts
    (64, 4, 2, 8, [32]),              # tiny drafter shape
    (128, 32, 8, 16, [2048, 2048]),   # full drafter head layout
    (128, 32, 8, 16, [2048, 100]),    # a short request: its last chunk holds only the block's keys
    (64, 4, 2, 8, [0, 0]),            # no context at all: one chunk of block keys
    # 32 requests x 8 KV heads: chunks of 9 tiles, taken by the 4-deep K/V ring; ragged
    # lengths, one empty context and one whole number of tiles
    (128, 32, 8, 16, [0, 1088] + [int(x) for x in np.random.default_rng(9).integers(500, 1100, 30)]),
])
def test_block_attention(D, NH, NKV, G, ctx):
    Bq = len(ctx)
    Lcap = max(max(ctx), 1) + 5
    Lmax = max(ctx)
    T = Bq * G
    qkvw = (NH + 2 * NKV) * D
    qkv = bf((T, qkvw), 41)
    K = bf((Bq, Lcap, NKV, D), 42)
    V = bf((Bq, Lcap, NKV, D), 43)
    ctx_len = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    out = torch.empty((T, NH * D), dtype=torch.bfloat16, device=DEV)
    ws = B.workspace(B.dfl_attention_workspace_bytes(Bq, G, NH, NKV, D, Lmax))
    flat = qkv.view(-1)   # k and v start inside each row; rows keep the qkv leading dimension
    B.dfl_block_attention(qkv, qkvw, flat[NH * D:], flat[(NH + NKV) * D:], qkvw, K, V, Lcap, Lmax,
                          ctx_len, Bq, G, NH, NKV, D, out, NH * D, ws)
    torch.cuda.synchronize()
    q_h = O.as_f64(h(qkv))
    q = q_h[:, :NH * D].reshape(Bq, G, NH, D)
    kb = q_h[:, NH * D:(NH + NKV) * D].reshape(Bq, G, NKV, D)
    vb = q_h[:, (NH + NKV) * D:].reshape(Bq, G, NKV, D)
    want = O.attention(q, h(K), h(V), kb, vb, np.array(ctx))
    assert_bf16_close(out.reshape(Bq, G, NH, D), want, "attention")


@pytest.mark.parametrize("M,N,K,out_f32", [
    (128, 6144, 5120, False),   # the fused q|k|v shape, split K
    (120, 1000, 1024, True),    # ragged N tile, fp32 out
    (7, 300, 128, False),       # ragged M and N, two groups
    (30, 520, 2048, True),      # two 16-row fragments, split K
    (50, 256, 640, False),      # four 16-row fragments
    (300, 32768, 256, True),    # 256 x 256 workgroup tiles, ragged M
    (600, 4096, 1024, False),   # 256 x 256 tiles with split K (too few tiles for a round)
    (512, 33024, 1024, True),   # a last round at most half full: 4-bit weights keep one launch
])
def test_linear_q4(M, N, K, out_f32):
    x = bf((M, K), 61)
    packed, sc, bi = synth.affine4_weight(N, K, seed=62, device=DEV)
    y = torch.empty((M, N), dtype=torch.float32 if out_f32 else torch.bfloat16, device=DEV)
    ws = B.workspace(B.dfl_linear_workspace_bytes(M, N, K))
    B.dfl_linear_q4(x, M, K, K, packed, sc, bi, N, y, N, out_f32, ws)
    torch.cuda.synchronize()
    w = O.dequant_affine4(packed.cpu().numpy(), h(sc), h(bi), bf16_weights=True)
    want = O.linear(h(x), w)
    (assert_f32_close if out_f32 else assert_bf16_close)(y, want, "4-bit affine projection")


@pytest.mark.parametrize("D,NH,NKV,G,ctx,pos,window", [
    (128, 32, 8, 16, [700, 2048], [700, 2048], 300),    # window inside one chunk, several tiles masked
    (128, 32, 8, 16, [5000, 129], [5000, 140], 2048),   # long context: earlier chunks skipped
    (64, 4, 2, 8, [40, 3], [45, 3], 5),                 # window < block: early rows see no context
    (64, 4, 2, 8, [33, 20], [33, 20], 100),             # a window wider than every context
    # the 4-deep K/V ring (32 requests x 8 KV heads, chunks of 9 tiles) under a window
    (128, 32, 8, 16, [int(x) for x in np.random.default_rng(10).integers(600, 1100, 32)],
     [int(x) for x in np.random.default_rng(10).integers(600, 1100, 32)], 700),
])
def test_block_attention_sliding_window(D, NH, NKV, G, ctx, pos, window):
    Bq = len(ctx)
    Lmax = max(ctx)
    Lcap = Lmax + 3
    T = Bq * G
    qkvw = (NH + 2 * NKV) * D
    qkv = bf((T, qkvw), 44)
    K = bf((Bq, Lcap, NKV, D), 45)
    V = bf((Bq, Lcap, NKV, D), 46)
    ctx_len = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    pos0 = torch.tensor(pos, dtype=torch.int32, device=DEV)
    out = torch.empty((T, NH * D), dtype=torch.bfloat16, device=DEV)
    ws = B.workspace(B.dfl_attention_workspace_bytes(Bq, G, NH, NKV, D, Lmax))
    flat = qkv.view(-1)
    B.dfl_block_attention(qkv, qkvw, flat[NH * D:], flat[(NH + NKV) * D:], qkvw, K, V, Lcap, Lmax,
                          ctx_len, Bq, G, NH, NKV, D, out, NH * D, ws, pos0=pos0, window=window)
    torch.cuda.synchronize()
    q_h = O.as_f64(h(qkv))
    q = q_h[:, :NH * D].reshape(Bq, G, NH, D)
    kb = q_h[:, NH * D:(NH + NKV) * D].reshape(Bq, G, NKV, D)
    vb = q_h[:, (NH + NKV) * D:].reshape(Bq, G, NKV, D)
    want = O.attention(q, h(K), h(V), kb, vb, np.array(ctx), np.array(pos), window)
    assert_bf16_close(out.reshape(Bq, G, NH, D), want, "sliding-window attention")


@pytest.mark.parametrize("T,H,G,grp", [(64, 512, 16, 16), (1024, 5120, 16, 16), (1024, 5120, 8, 16),
                                        (24, 256, 8, 16)])  # 1024 rows: 8-row workgroups, blocks of 16 and 8
def test_conv_prepare_finish(T, H, G, grp):
    x = bf((T, H), 51)
    kp = bf((4 * H // grp, H), 52, std=0.02)
    base = bf((2, 2, H), 53, 0.5, 0.1)
    y = bf((T, H), 54)
    res = bf((T, H), 55)
    a = torch.empty_like(x)
    coef1 = torch.empty((T, 2, H // grp), dtype=torch.float32, device=DEV)
    ws = B.workspace(B.dfl_conv_prepare_workspace_bytes(T, H, grp))
    B.dfl_conv_prepare(x, T, H, G, grp, kp, base, a, coef1, ws)
    f = torch.empty_like(x)
    B.dfl_conv_finish(y, coef1, base, T, H, G, grp, res, f)
    f0 = torch.empty_like(x)
    B.dfl_conv_finish(y, coef1, base, T, H, G, grp, None, f0)
    torch.cuda.synchronize()
    a_want, d1 = O.conv_prepare(h(x), h(kp), h(base), G, grp)
    assert_bf16_close(a, a_want, "conv prepare")
    assert_bf16_close(coef1, d1, "side-1 deltas")
    # finish on the GPU's own deltas isolates the conv from the projection's rounding
    f_want = O.conv_finish(h(y), h(coef1).astype(np.float64), h(base), G, grp)
    assert_bf16_close(f0, f_want, "conv finish")
    assert_bf16_close(f, O.as_f64(h(res)) + f_want, "conv finish + residual")


def test_conv_block_boundary_on_gpu():
    # perturbing the last row of block 0 leaves block 1 bit-identical (block locality)
    T, H, G, grp = 48, 512, 16, 16
    x = bf((T, H), 61)
    kp = bf((4 * H // grp, H), 62, std=0.02)
    base = bf((2, 2, H), 63, 0.5, 0.1)
    outs = []
    for bump in (0.0, 3.0):
        xx = x.clone()
        xx[G - 1] += bump
        a = torch.empty_like(xx)
        c1 = torch.empty((T, 2, H // grp), dtype=torch.float32, device=DEV)
        ws = B.workspace(B.dfl_conv_prepare_workspace_bytes(T, H, grp))
        B.dfl_conv_prepare(xx, T, H, G, grp, kp, base, a, c1, ws)
        f = torch.empty_like(xx)
        B.dfl_conv_finish(xx, c1, base, T, H, G, grp, None, f)
        outs.append((a, c1, f))
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.equal(outs[0][i][G:], outs[1][i][G:])
    assert not torch.equal(outs[0][0][:G], outs[1][0][:G])


@pytest.mark.parametrize("N,V,K,kind", [
    (7, 10000, 16, "normal"),      # ragged last chunk
    (5, 248320, 16, "normal"),     # full vocabulary
    (3, 1024, 4, "normal"),        # tiny vocabulary, one chunk
    (4, 9001, 16, "ties"),         # V not a multiple of 4, many equal values
    (2, 5000, 16, "constant"),     # every value equal: ids 0..K-1
    (3, 70, 32, "normal"),         # fewer elements than a chunk, K = 32
    (4, 248320, 16, "hot_tile"),   # every candidate inside one 256-column tile
    (3, 10000, 16, "hot_last"),    # maxima in the ragged last tile
    (3, 5000, 16, "neg_inf"),      # most of each row -inf: fewer finite tiles than K
    (2, 20000, 16, "theta_64"),    # exactly 64 values at or above theta: the gathered sort
    (2, 20000, 16, "theta_65"),    # 65 of them: the merging scan
])
def test_compute_candidates_bitexact(N, V, K, kind):
    g = torch.Generator(device=DEV).manual_seed(71)
    if kind == "normal":
        logits = torch.randn((N, V), generator=g, device=DEV) * 3
    elif kind == "ties":
        logits = torch.randint(-4, 5, (N, V), generator=g, device=DEV).float()
    elif kind == "hot_tile":
        logits = torch.randn((N, V), generator=g, device=DEV)
        for r in range(N):
            t = 37 * (r + 1) % (V // 256)
            logits[r, t * 256:(t + 1) * 256] += 20.0
    elif kind == "hot_last":
        logits = torch.randn((N, V), generator=g, device=DEV)
        logits[:, (V // 256) * 256:] += 20.0
    elif kind == "neg_inf":
        logits = torch.full((N, V), float("-inf"), device=DEV)
        logits[:, 300:310] = torch.randn((N, 10), generator=g, device=DEV)
        logits[:, 4000:4003] = 1.5
    elif kind.startswith("theta_"):
        # 16 tiles whose maximum is 10 (theta = 10, ties at theta inside them, ordered by
        # column), every other value below 1
        total = int(kind.split("_")[1])
        logits = torch.rand((N, V), generator=g, device=DEV)
        tiles = [3 + 4 * i for i in range(16)]
        for r in range(N):
            extra = total - 16
            for i, t in enumerate(tiles):
                n_here = 1 + extra // 16 + (1 if i < extra % 16 else 0)
                cols = t * 256 + (torch.arange(n_here, device=DEV) * 7 + 5 * r) % 256
                logits[r, cols] = 10.0
    else:
        logits = torch.full((N, V), 0.25, device=DEV)
    ids = torch.empty((N, K), dtype=torch.int32, device=DEV)
    vals = torch.empty((N, K), dtype=torch.float32, device=DEV)
    ws = B.workspace(B.dfl_candidates_workspace_bytes(N, V, K))
    B.dfl_compute_candidates(logits, N, V, K, ids, vals, ws)
    torch.cuda.synchronize()
    want_ids, want_vals = O.compute_candidates(logits.cpu().numpy(), K)
    assert np.array_equal(ids.cpu().numpy(), want_ids)
    assert np.array_equal(vals.cpu().numpy(), want_vals)


def _selector_inputs(Bq, S, K, R, V, seed, book_std=0.5):
    g = torch.Generator(device=DEV).manual_seed(seed)
    logits = torch.randn((Bq, S, V), generator=g, device=DEV) * 3
    pred = bf((V, R), seed + 1, std=book_std)
    succ = bf((V, R), seed + 2, std=book_std)
    z = torch.randn((Bq, S, R), generator=g, device=DEV)
    anchors = torch.randint(0, V, (Bq,), generator=g, device=DEV, dtype=torch.int32)
    cand_np, unary_np = O.compute_candidates(logits.cpu().numpy(), K)
    cand = torch.as_tensor(cand_np, device=DEV)
    unary = torch.as_tensor(unary_np, device=DEV)
    return logits, pred, succ, z, anchors, cand, unary


@pytest.mark.parametrize("Bq,S,K,R,V", [(3, 5, 16, 64, 5000), (1, 7, 4, 16, 1024), (2, 15, 32, 128, 300),
                                         (2, 6, 8, 12, 700)])   # R % 8 != 0: element gathers
def test_score_edges(Bq, S, K, R, V):
    _, pred, succ, z, anchors, cand, unary = _selector_inputs(Bq, S, K, R, V, 81)
    scores = torch.empty((Bq, S, K, K), dtype=torch.float32, device=DEV)
    B.dfl_score_edges(cand, unary, z, anchors, Bq, S, K, R, pred, succ, V, scores)
    torch.cuda.synchronize()
    want = O.score_edges(cand.cpu().numpy(), unary.cpu().numpy(), z.cpu().numpy().astype(np.float64),
                         anchors.cpu().numpy(), h(pred), h(succ))
    assert_f32_close(scores, want, "score_edges")
    s = scores.cpu().numpy()
    assert np.all(s[:, 0] == s[:, 0, :1]), "slot-0 rows must be identical across predecessors"


@pytest.mark.parametrize("Bq,S,K", [(32, 15, 16), (1, 7, 4), (3, 4, 32),
                                    (2, 20, 16), (2, 3, 64)])   # several LDS chunks of slots
def test_select_path_bitexact(Bq, S, K):
    g = torch.Generator().manual_seed(91)
    scores = (torch.randn((Bq, S, K, K), generator=g) * 2).float()
    scores[0, 0, 0, :2] = 5.0          # a tie: the lower slot must win
    cand = torch.randint(0, 100000, (Bq, S, K), generator=g, dtype=torch.int32)
    tokens = torch.empty((Bq, S), dtype=torch.int32, device=DEV)
    B.dfl_select_path(scores.to(DEV), cand.to(DEV), Bq, S, K, tokens)
    torch.cuda.synchronize()
    want = O.select_path(scores.numpy(), cand.numpy())
    assert np.array_equal(tokens.cpu().numpy(), want)


@pytest.mark.parametrize("N,H,R", [
    (120, 5120, 64),   # the full drafter's selector rows
    (37, 384, 20),     # ragged rows and columns; three K steps a quarter
    (5, 192, 8),       # H not a multiple of 128: the split-K GEMM
])
def test_selector_project(N, H, R):
    print(f"[selector_project] N={N} H={H} R={R}", flush=True)
    hh = bf((N, H), 101)
    proj = bf((R, H), 102, std=0.02)
    z = torch.empty((N, R), dtype=torch.float32, device=DEV)
    ws = B.workspace(B.dfl_selector_project_workspace_bytes(N, H, R))
    B.dfl_selector_project(hh, N, H, proj, R, z, ws)
    torch.cuda.synchronize()
    assert_bf16_close(z, O.selector_project(h(hh), h(proj)), "selector projection")
