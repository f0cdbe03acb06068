"""Convenience wrapper over the C ABI: allocates the caller-owned buffers (workspaces,
context K/V caches, outputs) with PyTorch and forwards to the binding."""
from __future__ import annotations

import torch

from . import binding as B_


class Drafter:
    def __init__(self, dims, weights: dict, tap_layer_ids=None, q4_weights=None):
        self.dims = dims
        self.handle = B_.dfl_drafter_load(dims, weights, tap_layer_ids, q4_weights=q4_weights)
        self._ws = None

    def close(self):
        if self.handle:
            B_.dfl_drafter_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def bind_target(self, lm_head: torch.Tensor, vocab_ids=None):
        """Copy the target's head once into the drafter's tile-contiguous layout (only the
        rows of a draft vocabulary, when vocab_ids lists one); draft() then accepts
        lm_head=None (or the same tensor) and streams the copy."""
        B_.dfl_bind_target(self.handle, lm_head, vocab_ids)
        self.head_cols = len(vocab_ids) if vocab_ids is not None else self.dims.vocab
        self._bound_ptr = lm_head.data_ptr()

    def alloc_kv(self, B: int, Lcap: int, device="cuda"):
        d = self.dims
        shape = (B, Lcap, d.kv_heads, d.head_dim)
        K = [torch.zeros(shape, dtype=torch.bfloat16, device=device) for _ in range(d.layers)]
        V = [torch.zeros(shape, dtype=torch.bfloat16, device=device) for _ in range(d.layers)]
        return K, V

    def materialize(self, taps: torch.Tensor, K: list, V: list, row_offset: int = 0):
        Bq, L = taps.shape[0], taps.shape[1]
        ws = B_.workspace(B_.dfl_context_workspace_bytes(self.handle, Bq, L))
        B_.dfl_context_materialize(self.handle, taps, Bq, L, row_offset, K[0].shape[1], K, V, ws)
        return ws

    def append(self, taps: torch.Tensor, row_offsets, starts, K: list, V: list):
        """Ragged append: taps [rows, n_taps*H] packs each request's new rows; request b's
        rows are taps[row_offsets[b]:row_offsets[b+1]], written from cache row starts[b]."""
        Bq = len(starts)
        ws = B_.workspace(B_.dfl_context_append_workspace_bytes(self.handle, Bq, int(row_offsets[-1])))
        B_.dfl_context_append(self.handle, taps, row_offsets, starts, Bq, K[0].shape[1], K, V, ws)
        return ws

    def workspace(self, B: int, G: int, Lmax: int) -> torch.Tensor:
        need = B_.dfl_draft_workspace_bytes(self.handle, B, G, Lmax)
        if self._ws is None or self._ws.numel() < need:
            self._ws = B_.workspace(need)
        return self._ws

    def draft(self, embeds, anchors, K, V, Lmax, ctx_len, pos0, lm_head, *, want_logits=False,
              tokens=None, logits=None, ws=None):
        Bq, G = embeds.shape[0], embeds.shape[1]
        Lcap = K[0].shape[1] if K else 0
        if tokens is None:
            tokens = torch.empty((Bq, G - 1), dtype=torch.int32, device=embeds.device)
        if want_logits and logits is None:
            bound = lm_head is None or lm_head.data_ptr() == getattr(self, "_bound_ptr", None)
            cols = getattr(self, "head_cols", self.dims.vocab) if bound else self.dims.vocab
            logits = torch.empty((Bq, G - 1, cols), dtype=torch.float32, device=embeds.device)
        ws = ws if ws is not None else self.workspace(Bq, G, Lmax)
        B_.dfl_draft_block(self.handle, embeds, anchors, Bq, G, K, V, Lcap, Lmax, ctx_len, pos0, lm_head,
                           tokens, logits, ws)
        return (tokens, logits) if want_logits else tokens
