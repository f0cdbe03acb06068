"""dfl_compute_candidates_static (no workspace, a static device scratch) against
dfl_compute_candidates (caller workspace), bit for bit, on two calls in a row whose second
input is smaller, so a stale tail of the first call's tile maxima stays in the scratch."""
import numpy as np
import pytest
import torch

from dflash2_block_drafter_amd import binding as B
from dflash2_block_drafter_amd import synth
from oracle import dflash2 as O

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(logits, N, V, K):
    ids_w = torch.full((N, K), -1, dtype=torch.int32, device=DEV)
    un_w = torch.full((N, K), float("nan"), dtype=torch.float32, device=DEV)
    ws = B.workspace(B.dfl_candidates_workspace_bytes(N, V, K))
    B.dfl_compute_candidates(logits, N, V, K, ids_w, un_w, ws)
    ids_s = torch.full((N, K), -1, dtype=torch.int32, device=DEV)
    un_s = torch.full((N, K), float("nan"), dtype=torch.float32, device=DEV)
    B.dfl_compute_candidates_static(logits, N, V, K, ids_s, un_s)
    torch.cuda.synchronize()
    return ids_w, un_w, ids_s, un_s


def test_static_scratch_candidates_match_workspace_call():
    # 1: the selector workload's 480 rows over V = 248320 (465,600 tile maxima); 2: fewer rows
    # with ties (a quarter of each row's values repeat one level), a ragged last tile
    cases = [(480, 248320, 16, 0), (37, 10001, 16, 1)]
    for N, V, K, ties in cases:
        print(f"[no-alloc] N={N} V={V} K={K} ties={ties}", flush=True)
        lg = synth.normal((N, V), 0.0, 3.0, seed=4000 + N, device=DEV, dtype=torch.float32)
        if ties:
            lg[:, ::4] = 2.5
        ids_w, un_w, ids_s, un_s = _both(lg, N, V, K)
        assert torch.equal(ids_w, ids_s) and torch.equal(un_w, un_s)
        rows = np.arange(0, N, max(1, N // 8))
        want_ids, want_un = O.compute_candidates(lg.cpu().numpy()[rows], K)
        assert np.array_equal(ids_s.cpu().numpy()[rows], want_ids)
        assert np.array_equal(un_s.cpu().numpy()[rows], want_un)
